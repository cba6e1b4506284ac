"""qdec_op_attention_noalloc (split-KV partials in the library's static device scratch, no
workspace argument, nothing allocated) against qdec_op_attention on the same inputs.

Two calls in a row, the second with a smaller input (fewer positions, other head counts), each
compared bit for bit with the workspace entry point's output (the same kernels, partition
lengths and merge order) and with the two-pass oracle (max-abs 1e-4, the fp32 budget).  A call
whose partials would not fit the 16 MiB scratch is rejected with QDEC_E_RANGE and enqueues
nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_step_04_amd import qdec as Q
from decode_step_04_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _paged(kl, vl, bt, num_pages):
    kb, vb = synth.bf16_to_bits(kl), synth.bf16_to_bits(vl)
    kp = oracle.pool_scatter(kb, 0, bt, num_pages, 16)
    vp = oracle.pool_scatter(vb, 0, bt, num_pages, 16)
    kp = torch.from_numpy(kp.view(np.int16)).view(torch.bfloat16).to(DEV)
    vp = torch.from_numpy(vp.view(np.int16)).view(torch.bfloat16).to(DEV)
    return kp, vp


def _case(T, hq, hkv, d, part, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((hq, d), generator=g, device=DEV) * 0.5
    kl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    n_pages = (T + 15) // 16
    bt = np.random.default_rng(seed).permutation(n_pages + 2)[:n_pages].astype(np.int32)
    kp, vp = _paged(kl, vl, bt, n_pages + 2)
    return q, kl, vl, kp, vp, torch.from_numpy(bt).to(DEV)


def _both(q, kp, vp, btd, T, hq, hkv, d, part):
    ws_bytes = Q.qdec_op_attention_workspace(T, hq, d, part)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    ref = torch.empty((hq, d), device=DEV)
    got = torch.full((hq, d), float("nan"), device=DEV)
    Q.qdec_op_attention(q, Q.F32, kp, vp, Q.BF16, btd, T, hq, hkv, d, part, ws, ws.numel(), ref,
                        Q.F32)
    Q.qdec_op_attention_noalloc(q, Q.F32, kp, vp, Q.BF16, btd, T, hq, hkv, d, part, got, Q.F32)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_attention_matches_workspace_entry_point_twice():
    cases = [(32768, 32, 8, 128, 0, 1),      # 8 x 64 partitions of 512 positions
             (1000, 16, 2, 64, 64, 2)]       # then a smaller call: 16 partitions, other heads
    for T, hq, hkv, d, part, seed in cases:
        print(f"noalloc attention T={T} hq={hq} hkv={hkv} d={d} part={part}", flush=True)
        q, kl, vl, kp, vp, btd = _case(T, hq, hkv, d, part, seed)
        got, ref = _both(q, kp, vp, btd, T, hq, hkv, d, part)
        np.testing.assert_array_equal(got, ref)
        exact = oracle.attention(q.cpu().numpy().astype(np.float64), kl.float().cpu().numpy(),
                                 vl.float().cpu().numpy())
        assert np.max(np.abs(got - exact)) <= 1e-4


def test_noalloc_attention_single_partition_and_rejection():
    q, kl, vl, kp, vp, btd = _case(40, 8, 8, 128, 0, 3)
    got, ref = _both(q, kp, vp, btd, 40, 8, 8, 128, 0)          # one partition: no scratch
    np.testing.assert_array_equal(got, ref)
    # 64 query heads x 8192 partitions of 64 positions x 130 floats: 272 MB of partials
    out = torch.empty((64, 128), device=DEV)
    with pytest.raises(Q.QdecError) as e:
        Q.qdec_op_attention_noalloc(q, Q.F32, kp, vp, Q.BF16, btd, 64 * 8192, 64, 8, 128, 64, out,
                                    Q.F32)
    assert e.value.status == Q.E_RANGE
