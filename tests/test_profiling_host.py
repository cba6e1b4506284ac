"""Host logic of the profile summaries (no GPU): the copy / compute overlap of two interval
sets, checked on hand-computed cases."""
from decode_step_04_amd import profiling as P


def test_overlap_hand_computed():
    k = [(0, 10), (12, 20), (25, 40)]
    c = [(5, 15), (30, 50)]
    r = P.overlap(k, c, skip=0)
    # window 5..50; kernels busy 5+8+15 = 28, copies 10+20 = 30, both 5+3+10 = 18
    assert r["window_us"] * 1e3 == 45
    assert round(r["kernel_busy_us"] * 1e3) == 28 and round(r["copy_busy_us"] * 1e3) == 30
    assert round(r["both_busy_us"] * 1e3) == 18
    assert abs(r["copy_hidden_under_kernels"] - 0.6) < 1e-12
    assert abs(r["either_busy_frac"] - 40 / 45) < 1e-12


def test_overlap_disjoint_nested_and_skip():
    assert P.overlap([(0, 5)], [(10, 20)], skip=0)["both_busy_us"] == 0
    r = P.overlap([(0, 100)], [(10, 20), (15, 30), (40, 50)], skip=0)   # copies nested in a kernel
    assert round(r["copy_busy_us"] * 1e3) == 30 and r["copy_hidden_under_kernels"] == 1.0
    r = P.overlap([(0, 100)], [(0, 10), (90, 100)], skip=0.5)          # first half dropped
    assert round(r["window_us"] * 1e3) == 50 and round(r["copy_busy_us"] * 1e3) == 10
    assert P.overlap([(0, 1)], []) is None
