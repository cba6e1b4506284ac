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
          (2048, 4096, 1024), (130, 6144, 1024), (2000, 4300, 1024), (300, 96, 96)]


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


@pytest.mark.parametrize("m,n,k", [(3, 48, 96), (300, 1024, 2048), (64, 4096, 4096),
                                   (2048, 4096, 1024), (1999, 4200, 512)])
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


@pytest.mark.parametrize("m,f,k", [(2, 64, 64), (77, 200, 1024), (512, 3072, 1024),
                                   (2048, 3072, 1024), (2001, 3000, 1024)])
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


# ---- the whole prefill at the Qwen3-0.6B shape ------------------------------------------------------

from decode_step_04_amd import loader  # noqa: E402

SHAPE = synth.QWEN3_0P6B


class PrefillSetup:
    """bf16 weights and KV, the 16-bit activation policy (what prefill computes), an empty cache
    of max_context positions behind a random block table, and the oracle model on the same
    weights."""

    def __init__(self, max_context=1024, max_prefill=256):
        print(f"prefill setup max_context={max_context} max_prefill={max_prefill}", flush=True)
        n_pages = max_context // 16
        self.cfg = loader.config_for(SHAPE, path="bf16", num_pages=n_pages, max_context=max_context,
                                     act="bf16", max_prefill=max_prefill)
        self.ctx = Q.qdec_create(self.cfg, 0)
        w = synth.bf16_model(SHAPE, seed=0, device=DEV)
        loader.upload_weights(self.ctx, w, DEV)
        self.table = synth.block_table(n_pages, n_pages, seed=2)
        Q.qdec_kv_set_block_table(self.ctx, self.table)
        self.hw = synth.host_weights(w)
        del w
        self.om = oracle.Model(dict(SHAPE, act_bf16=1, kv_bf16=1, logits_bf16=1), self.hw,
                               max_ctx=max_context)
        self.hidden = torch.empty(SHAPE["hidden"], device=DEV)
        self.logits = torch.empty(SHAPE["vocab"], dtype=torch.bfloat16, device=DEV)
        self.amax = torch.empty(1, dtype=torch.int32, device=DEV)

    def prefill(self, tokens, pos0):
        t = torch.from_numpy(tokens).to(DEV)
        Q.qdec_prefill(self.ctx, t, len(tokens), pos0, self.hidden, self.logits, self.amax)
        torch.cuda.synchronize()
        return (self.hidden.cpu().numpy().astype(np.float64),
                synth.bf16_to_f32(self.logits).astype(np.float64), int(self.amax.item()))

    def oracle_run(self, tokens, pos0):
        """(plain-fp32 oracle, fp64 oracle) results of the last token after decoding `tokens` one
        by one from pos0; the fp64 pass runs last so the oracle's cache holds its rows."""
        with oracle.fp32_arithmetic():
            for i, tok in enumerate(tokens):
                r32 = self.om.step(pos0 + i, token=int(tok))
        for i, tok in enumerate(tokens):
            r64 = self.om.step(pos0 + i, token=int(tok))
        return r32, r64

    def close(self):
        Q.qdec_destroy(self.ctx)


def _check_bf16_policy(got, ref, ref32, what):
    gh, gl, ga = got
    rh, rl, ra = ref
    rel = np.linalg.norm(gh - rh) / np.linalg.norm(rh)
    lmax = np.max(np.abs(gl - rl))
    d32 = np.linalg.norm(ref32[0] - rh) / np.linalg.norm(rh)
    l32 = np.max(np.abs(ref32[1] - rl))
    print(f"{what}: hidden rel-L2 {rel:.3e} logits max-abs {lmax:.3e} argmax {ga} vs {ra} "
          f"(plain-fp32 oracle: {d32:.3e}, {l32:.3e})", flush=True)
    assert rel <= max(1.5e-2, 2 * d32)
    assert lmax <= max(5e-2, 2 * l32)
    assert rl[ga] >= rl.max() - 2 * 2.0**-8 * abs(rl.max()) - 2 * l32


def _check_kv(s, layer, n):
    """The cache rows the prefill wrote against the oracle's (both bf16 values)."""
    hkv, d = SHAPE["n_kv_heads"], SHAPE["head_dim"]
    k = torch.empty((n, hkv, d), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((n, hkv, d), dtype=torch.bfloat16, device=DEV)
    Q.qdec_kv_read(s.ctx, layer, 0, n, k, v)
    torch.cuda.synchronize()
    for got, ref in ((k.float().cpu().numpy(), s.om.k_cache[layer][:n]),
                     (v.float().cpu().numpy(), s.om.v_cache[layer][:n])):
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel <= 2e-2, (layer, rel)


@pytest.mark.timeout(600)
def test_prefill_matches_token_by_token_decode():
    """One prefill of 100 tokens, then a second of 37 at pos0 = 100 (queries over cached keys),
    then a decode step at pos 137: each against the oracle decoding the same tokens one by one
    under the same 16-bit activation policy; the cache rows the prefill wrote against the
    oracle's."""
    s = PrefillSetup()
    try:
        toks = synth.prompt_tokens(SHAPE["vocab"], 137, seed=4)
        got = s.prefill(toks[:100], 0)
        r32, r64 = s.oracle_run(toks[:100], 0)
        _check_bf16_policy(got, r64, r32, "prefill 100")
        _check_kv(s, 0, 100)
        _check_kv(s, SHAPE["n_layers"] - 1, 100)
        got = s.prefill(toks[100:], 100)
        r32, r64 = s.oracle_run(toks[100:], 100)
        _check_bf16_policy(got, r64, r32, "prefill 37 at 100")
        # a decode step continues from the prefilled cache
        tok = torch.tensor([int(toks[-1])], dtype=torch.int32, device=DEV)
        st = Q.make_step(137, token_id=tok, hidden_out=s.hidden, logits_out=s.logits,
                         argmax_out=s.amax)
        Q.qdec_decode_step(s.ctx, st)
        torch.cuda.synchronize()
        got = (s.hidden.cpu().numpy().astype(np.float64),
               synth.bf16_to_f32(s.logits).astype(np.float64), int(s.amax.item()))
        r32, r64 = s.oracle_run(toks[-1:], 137)
        _check_bf16_policy(got, r64, r32, "decode at 137")
        assert Q.qdec_device_error(s.ctx) == 0
    finally:
        s.close()


def test_prefill_rejects_bad_calls():
    s = PrefillSetup(max_context=256, max_prefill=32)
    try:
        t = torch.zeros(64, dtype=torch.int32, device=DEV)
        with pytest.raises(Q.QdecError):
            Q.qdec_prefill(s.ctx, t, 33, 0)            # above max_prefill
        with pytest.raises(Q.QdecError):
            Q.qdec_prefill(s.ctx, t, 0, 0)             # empty
        with pytest.raises(Q.QdecError):
            Q.qdec_prefill(s.ctx, t, 8, 250)           # past max_context
    finally:
        s.close()
