"""Pins of the oracle's group-wise int8 / int4 formats (runs without a GPU).

[Qwen3-runtime] §13.1 keeps one scale per 128-value group of a row and forms each group's
integer-weighted partial sum before multiplying it by the group's scale; [ETE] names 4-bit codes
as the next step after per-row int8.  The pins: codes and scales recovered exactly from weights
built as code x power-of-two scale (a closed form), the per-element error bound, group
independence, the reduction of a one-group row to the per-row quantiser, and the GEMV against
numpy on dequantised weights.  The int4 nibbles are unpacked here with numpy, independently of
the oracle's C code.
"""
import numpy as np
import pytest

import oracle

G = 128


def unpack_int4(packed):
    """[n, k/2] uint8 -> [n, k] int codes: element 2j in the low nibble of byte j, code + 8."""
    lo = (packed & 0x0F).astype(np.int64) - 8
    hi = (packed >> 4).astype(np.int64) - 8
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def codes_of(q, bits):
    return q.astype(np.int64) if bits == 8 else unpack_int4(q)


def dequant(q, s, bits):
    return codes_of(q, bits).astype(np.float64) * np.repeat(s.astype(np.float64), G, axis=1)


@pytest.mark.parametrize("bits", [8, 4])
def test_known_codes_and_scales_are_recovered_exactly(bits):
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(40 + bits)
    n, k = 6, 4 * G
    ng = k // G
    codes = rng.integers(-qmax, qmax + 1, size=(n, k))
    exps = rng.integers(-12, -2, size=(n, ng))
    # every group reaches +-qmax once, so max|w| / qmax is the power of two exactly
    for r in range(n):
        for g in range(ng):
            codes[r, g * G + rng.integers(0, G)] = qmax if rng.random() < 0.5 else -qmax
    codes[2, G:2 * G] = 0                        # an all-zero group
    scale = np.ldexp(1.0, exps).astype(np.float32)
    scale[2, 1] = 0.0
    w = (codes * np.repeat(scale.astype(np.float64), G, axis=1)).astype(np.float32)
    q, s = oracle.quantize_groups(w, bits)
    assert q.shape == ((n, k) if bits == 8 else (n, k // 2))
    np.testing.assert_array_equal(s, scale)
    np.testing.assert_array_equal(codes_of(q, bits), codes)
    if bits == 4:
        # storage: offset-binary nibbles, even element low; code -7..7 never makes nibble 0
        assert np.all((q & 0x0F) >= 1) and np.all((q >> 4) >= 1)


@pytest.mark.parametrize("bits", [8, 4])
def test_error_bound_extremes_and_group_independence(bits):
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(50 + bits)
    n, k = 16, 6 * G
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[4, 3 * G:4 * G] = 0.0
    w[7, 5 * G + 9] = -0.75                      # dominant negative entry in the last group
    q, s = oracle.quantize_groups(w, bits)
    c = codes_of(q, bits)
    assert np.all(np.abs(c) <= qmax)
    grp_max = np.abs(c).reshape(n, k // G, G).max(axis=2)
    nz = np.abs(w).reshape(n, k // G, G).max(axis=2) > 0
    assert np.all(grp_max[nz] == qmax) and np.all(grp_max[~nz] == 0)
    assert s[4, 3] == 0 and c[7, 5 * G + 9] == -qmax
    err = np.abs(dequant(q, s, bits) - w)
    bound = np.repeat(s.astype(np.float64), G, axis=1) * 0.5 * (1 + 1e-6) + 1e-30
    assert np.all(err <= bound)
    # the scale really is per group: group 2 of row 0 rescaled alone changes only its own codes
    w2 = w.copy()
    w2[0, 2 * G:3 * G] *= 3.0
    q2, s2 = oracle.quantize_groups(w2, bits)
    c2 = codes_of(q2, bits)
    same = np.ones(k // G, dtype=bool)
    same[2] = False
    np.testing.assert_array_equal(s2[0, same], s[0, same])
    np.testing.assert_array_equal(s2[1:], s[1:])
    mask = np.repeat(same, G)
    np.testing.assert_array_equal(c2[0, mask], c[0, mask])
    assert s2[0, 2] != s[0, 2]


def test_one_group_row_reduces_to_the_per_row_quantiser():
    rng = np.random.default_rng(60)
    w = (rng.standard_normal((32, G)) * 0.05).astype(np.float32)
    q8, s8 = oracle.quantize_groups(w, 8)
    qr, sr = oracle.quantize_rows(w)
    np.testing.assert_array_equal(q8, qr)
    np.testing.assert_array_equal(s8[:, 0], sr)


@pytest.mark.parametrize("bits", [8, 4])
def test_group_gemv_matches_numpy_on_dequantised_weights(bits):
    rng = np.random.default_rng(70 + bits)
    n, k = 29, 5 * G
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal(k)
    q, s = oracle.quantize_groups(w, bits)
    ref = dequant(q, s, bits) @ x
    got = oracle.gemv(q, x, s)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)
    # one scale per row (group 0's) is a different function: the pin sees it
    wrong = codes_of(q, bits).astype(np.float64) @ x * s[:, 0].astype(np.float64)
    assert not np.allclose(got, wrong, rtol=1e-6)
    # and the int4 element order matters (swapping the nibbles of every byte breaks it)
    if bits == 4:
        swapped = ((q & 0x0F) << 4) | (q >> 4)
        assert not np.allclose(oracle.gemv(swapped.astype(np.uint8), x, s), ref, rtol=1e-6)


def _f32(v):
    return float(np.float32(v))


@pytest.mark.parametrize("bits", [8, 4])
def test_fp32_mode_group_gemv_is_sequential_fp32(bits):
    rng = np.random.default_rng(80 + bits)
    n, k = 3, 2 * G
    w = (rng.standard_normal((n, k)) * 0.1).astype(np.float32)
    x = rng.standard_normal(k).astype(np.float32)
    q, s = oracle.quantize_groups(w, bits)
    with oracle.fp32_arithmetic():
        got = oracle.gemv(q, x, s)
    c = codes_of(q, bits)
    for r in range(n):
        total = 0.0
        for g in range(k // G):
            part = 0.0
            for j in range(g * G, (g + 1) * G):
                part = _f32(part + float(c[r, j]) * float(x[j]))
            total = _f32(total + _f32(part * float(s[r, g])))
        assert got[r] == total, r
