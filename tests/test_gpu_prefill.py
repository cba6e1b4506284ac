"""Prefill kernels (through the C ABI) against the CPU oracle.

The prefill GEMM takes bf16 operands on the matrix cores with fp32 accumulation; its reference is
the oracle's GEMV applied to each row of A (exact fp64 dot products of the same bf16 values).
Bars: fp32 outputs max-abs <= 1e-4 (fp32 accumulation over k <= 3072 of terms ~0.02); bf16
outputs within one bf16 ulp of the exact value plus 1e-6.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_step_04_amd import qdec as Q
from decode_step_04_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return synth.bf16_to_bits(t)


def _rows_exact(a_bits, w_bits, rows):
    """exact[r] = W . A[r] for the sampled rows r (fp64, the oracle's GEMV)."""
    return np.stack([oracle.gemv(w_bits, oracle.bf16_bits_to_f64(a_bits[r])) for r in rows])


def _bf16_ulp_ok(got, exact, extra=1e-6):
    return np.abs(got - exact) <= np.abs(exact) * 2.0**-8 + extra


SHAPES = [(1, 16, 32), (5, 33, 64), (128, 128, 128), (200, 300, 1024), (17, 1024, 3072),
          (2048, 4096, 1024), (130, 6144, 1024)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_store_matches_oracle(m, n, k):
    print(f"gemm store m={m} n={n} k={k}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(m * 131 + n * 7 + k)
    a = torch.randn((m, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    y32 = torch.empty((m, n), device=DEV)
    ybf = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    Q.qdec_op_gemm(a, w, y32, Q.F32, None, Q.GEMM_STORE, m, n, k)
    Q.qdec_op_gemm(a, w, ybf, Q.BF16, None, Q.GEMM_STORE, m, n, k)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(1).choice(m, min(m, 48), replace=False),
                                     [0, m - 1]]))
    exact = _rows_exact(_bits(a), _bits(w), rows)
    assert np.max(np.abs(y32.cpu().numpy()[rows] - exact)) <= 1e-4
    assert _bf16_ulp_ok(synth.bf16_to_f32(ybf)[rows], exact).all()


@pytest.mark.parametrize("m,n,k", [(3, 48, 96), (300, 1024, 2048), (64, 4096, 4096)])
def test_gemm_resid_adds_into_the_stream(m, n, k):
    g = torch.Generator(device=DEV).manual_seed(m + n + k)
    a = torch.randn((m, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    r0 = torch.randn((m, n), generator=g, device=DEV)
    r = r0.clone()
    Q.qdec_op_gemm(a, w, None, Q.F32, r, Q.GEMM_RESID, m, n, k)
    torch.cuda.synchronize()
    rows = np.unique([0, m // 2, m - 1])
    exact = _rows_exact(_bits(a), _bits(w), rows) + r0.cpu().numpy()[rows].astype(np.float64)
    assert np.max(np.abs(r.cpu().numpy()[rows] - exact)) <= 1e-4


@pytest.mark.parametrize("m,f,k", [(2, 64, 64), (77, 200, 1024), (512, 3072, 1024)])
def test_gemm_swiglu_epilogue(m, f, k):
    g = torch.Generator(device=DEV).manual_seed(m * 3 + f + k)
    a = torch.randn((m, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((2 * f, k), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    y = torch.empty((m, f), device=DEV, dtype=torch.bfloat16)
    Q.qdec_op_gemm(a, w, y, Q.BF16, None, Q.GEMM_SWIGLU, m, f, k)
    torch.cuda.synchronize()
    rows = np.unique([0, m // 3, m - 1])
    gu = _rows_exact(_bits(a), _bits(w), rows)
    exact = oracle.silu(gu[:, :f]) * gu[:, f:]
    assert _bf16_ulp_ok(synth.bf16_to_f32(y)[rows], exact, extra=1e-5).all()


def test_gemm_rejects_bad_arguments():
    a = torch.zeros((4, 64), device=DEV, dtype=torch.bfloat16)
    w = torch.zeros((8, 64), device=DEV, dtype=torch.bfloat16)
    y = torch.zeros((4, 8), device=DEV)
    with pytest.raises(Q.QdecError):
        Q.qdec_op_gemm(a, w, y, Q.F32, None, Q.GEMM_STORE, 4, 8, 48)       # k % 32
    with pytest.raises(Q.QdecError):
        Q.qdec_op_gemm(a, w, y, Q.F32, None, Q.GEMM_SWIGLU, 4, 4, 64)      # SwiGLU writes bf16
    with pytest.raises(Q.QdecError):
        Q.qdec_op_gemm(a, w, None, Q.F32, None, Q.GEMM_RESID, 4, 8, 64)    # no residual


# ---- causal prefill attention -------------------------------------------------------------------------

def _paged_bf16(kl, vl, bt, num_pages):
    """Pool tensors holding logical bf16 K/V [T, Hkv, D] through block table bt (the oracle's
    placement, bit for bit)."""
    kp = oracle.pool_scatter(synth.bf16_to_bits(kl), 0, bt, num_pages, 16)
    vp = oracle.pool_scatter(synth.bf16_to_bits(vl), 0, bt, num_pages, 16)
    kp = torch.from_numpy(kp.view(np.int16)).view(torch.bfloat16)
    vp = torch.from_numpy(vp.view(np.int16)).view(torch.bfloat16)
    return kp.to(DEV), vp.to(DEV)


@pytest.mark.parametrize("d,hq,hkv", [(128, 16, 8), (128, 32, 8), (64, 4, 2), (128, 8, 8),
                                      (128, 24, 8), (64, 16, 2), (128, 4, 1)])
@pytest.mark.parametrize("pos0,P", [(0, 1), (0, 17), (0, 64), (5, 40), (100, 33), (0, 300),
                                    (1000, 129)])
def test_prefill_attention_matches_oracle(d, hq, hkv, pos0, P):
    """Query t sees keys 0 .. pos0 + t.  The reference is the oracle's two-pass fp64 attention
    of the same bf16 q, K and V per query.  Bar: the output is rounded to bf16 and the
    probabilities are rounded to bf16 as the second product's operand, so |got - ref| <=
    2^-7 |ref| + 4e-3 (values ~N(0, 1))."""
    print(f"prefill attention d={d} hq={hq} hkv={hkv} pos0={pos0} P={P}", flush=True)
    T = pos0 + P
    g = torch.Generator(device=DEV).manual_seed(T * 7 + d + hq + P)
    q = (torch.randn((P, hq, d), generator=g, device=DEV) * 0.5).to(torch.bfloat16)
    kl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    n_pages = (T + 15) // 16
    num_pages = n_pages + 3
    bt = np.random.default_rng(T).permutation(num_pages)[:n_pages].astype(np.int32)
    kp, vp = _paged_bf16(kl, vl, bt, num_pages)
    out = torch.empty((P, hq, d), device=DEV, dtype=torch.bfloat16)
    Q.qdec_op_prefill_attention(q, kp, vp, torch.from_numpy(bt).to(DEV), pos0, P, hq, hkv, d, out)
    torch.cuda.synchronize()
    got = synth.bf16_to_f32(out).astype(np.float64)
    qh = synth.bf16_to_f32(q).astype(np.float64)
    kh, vh = kl.float().cpu().numpy(), vl.float().cpu().numpy()
    ts = np.unique(np.concatenate([np.random.default_rng(P).choice(P, min(P, 24), replace=False),
                                   [0, P - 1]]))
    for t in ts:
        ref = oracle.attention(qh[t], kh[: pos0 + t + 1], vh[: pos0 + t + 1])
        err = np.abs(got[t] - ref)
        assert np.all(err <= 2.0**-7 * np.abs(ref) + 4e-3), (t, float(err.max()))
