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
    rows = np.arange(m)                          # every row, every column
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
    rows = np.arange(m)                          # every row, every column
    gu = _rows_exact(_bits(a), _bits(w), rows)
    exact = oracle.silu(gu[:, :f]) * gu[:, f:]
    assert _bf16_ulp_ok(synth.bf16_to_f32(y)[rows], exact, extra=1e-5).all()


# Products with at least 512 tiles of 256 x 256 run on the direct-to-LDS kernel (8 waves, swizzled
# LDS stages); these shapes reach it, with ragged rows and columns.  Sampled rows, every column.
def _sample_rows(m, n_rows=40, seed=2):
    return np.unique(np.concatenate([np.random.default_rng(seed).choice(m, min(m, n_rows), replace=False),
                                     [0, m - 1]]))


@pytest.mark.parametrize("m,n,k", [(2048, 16384, 512), (2000, 16400, 256)])
def test_gemm_large_tiles_store_and_resid(m, n, k):
    print(f"gemm large tiles m={m} n={n} k={k}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(m + 3 * n + k)
    a = torch.randn((m, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    y32 = torch.empty((m, n), device=DEV)
    ybf = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    r0 = torch.randn((m, n), generator=g, device=DEV)
    r = r0.clone()
    Q.qdec_op_gemm(a, w, y32, Q.F32, None, Q.GEMM_STORE, m, n, k)
    Q.qdec_op_gemm(a, w, ybf, Q.BF16, None, Q.GEMM_STORE, m, n, k)
    Q.qdec_op_gemm(a, w, None, Q.F32, r, Q.GEMM_RESID, m, n, k)
    torch.cuda.synchronize()
    rows = _sample_rows(m)
    exact = _rows_exact(_bits(a), _bits(w), rows)
    assert np.max(np.abs(y32.cpu().numpy()[rows] - exact)) <= 1e-4
    assert _bf16_ulp_ok(synth.bf16_to_f32(ybf)[rows], exact).all()
    resid_exact = exact + r0.cpu().numpy()[rows].astype(np.float64)
    assert np.max(np.abs(r.cpu().numpy()[rows] - resid_exact)) <= 1e-4


@pytest.mark.parametrize("m,f,k", [(2001, 8200, 512), (2048, 12288, 4096)])
def test_gemm_large_tiles_swiglu(m, f, k):
    """Includes the 8B-class prefill's gate-up product (2048 tokens, FFN 12288, hidden 4096)."""
    print(f"gemm large tiles swiglu m={m} f={f} k={k}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(m * 5 + f + k)
    a = torch.randn((m, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((2 * f, k), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    y = torch.empty((m, f), device=DEV, dtype=torch.bfloat16)
    Q.qdec_op_gemm(a, w, y, Q.BF16, None, Q.GEMM_SWIGLU, m, f, k)
    torch.cuda.synchronize()
    rows = _sample_rows(m, 24)
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
    _check_prefill_attention(d, hq, hkv, pos0, P)


@pytest.mark.parametrize("d,hq,hkv", [(128, 16, 8), (128, 32, 8)])
@pytest.mark.parametrize("pos0,P", [(0, 2048), (3000, 1000), (0, 4097)])
def test_prefill_attention_long_prompts(d, hq, hkv, pos0, P):
    """Prompts of many query blocks (paired heavy with light in one work-group) over contexts
    of several page chunks, at the same bar."""
    _check_prefill_attention(d, hq, hkv, pos0, P)


def _check_prefill_attention(d, hq, hkv, pos0, P):
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
# the same widths with 2 layers: the first two layers of the 28-layer model (same draw order)
SHAPE2 = dict(SHAPE, name="qwen3-0.6b-shape-2-layers", n_layers=2)


class PrefillSetup:
    """bf16 weights and KV, the 16-bit activation policy (what prefill computes), an empty cache
    of max_context positions behind a random block table, and the oracle model on the same
    weights."""

    def __init__(self, shape=SHAPE, max_context=1024, max_prefill=256, oracle_model=True):
        print(f"prefill setup {shape['name']} max_context={max_context} "
              f"max_prefill={max_prefill}", flush=True)
        self.shape = shape
        n_pages = max_context // 16
        self.cfg = loader.config_for(shape, path="bf16", num_pages=n_pages, max_context=max_context,
                                     act="bf16", max_prefill=max_prefill)
        self.ctx = Q.qdec_create(self.cfg, 0)
        w = synth.bf16_model(shape, seed=0, device=DEV)
        loader.upload_weights(self.ctx, w, DEV)
        self.table = synth.block_table(n_pages, n_pages, seed=2)
        Q.qdec_kv_set_block_table(self.ctx, self.table)
        self.hw = synth.host_weights(w) if oracle_model else None
        del w
        self.om = oracle.Model(dict(shape, act_bf16=1, kv_bf16=1, logits_bf16=1), self.hw,
                               max_ctx=max_context) if oracle_model else None
        self.hidden = torch.empty(shape["hidden"], device=DEV)
        self.logits = torch.empty(shape["vocab"], dtype=torch.bfloat16, device=DEV)
        self.amax = torch.empty(1, dtype=torch.int32, device=DEV)

    def prefill(self, tokens, pos0):
        t = torch.from_numpy(tokens).to(DEV)
        Q.qdec_prefill(self.ctx, t, len(tokens), pos0, self.hidden, self.logits, self.amax)
        torch.cuda.synchronize()
        return (self.hidden.cpu().numpy().astype(np.float64),
                synth.bf16_to_f32(self.logits).astype(np.float64), int(self.amax.item()))

    def oracle_run(self, tokens, pos0, fp32_pass=True):
        """(plain-fp32 oracle or None, fp64 oracle) results of the last token after decoding
        `tokens` one by one from pos0 (logits for the last token only); the fp64 pass runs last
        so the oracle's cache holds its rows."""
        r32 = None
        last = len(tokens) - 1
        if fp32_pass:
            with oracle.fp32_arithmetic():
                for i, tok in enumerate(tokens):
                    r32 = self.om.step(pos0 + i, token=int(tok), want_logits=i == last)
        for i, tok in enumerate(tokens):
            r64 = self.om.step(pos0 + i, token=int(tok), want_logits=i == last)
        return r32, r64

    def kv_rows(self, layer, n):
        hkv, d = self.shape["n_kv_heads"], self.shape["head_dim"]
        k = torch.empty((n, hkv, d), dtype=torch.bfloat16, device=DEV)
        v = torch.empty((n, hkv, d), dtype=torch.bfloat16, device=DEV)
        Q.qdec_kv_read(self.ctx, layer, 0, n, k, v)
        torch.cuda.synchronize()
        return k.float().cpu().numpy(), v.float().cpu().numpy()

    def close(self):
        Q.qdec_destroy(self.ctx)


def _fixed_bar(got, ref, what):
    """The fixed bar of the bf16 path: hidden relative L2 <= 1.5e-2, logits max-abs <= 5e-2, and
    the greedy id a maximiser of the oracle's logits up to bf16 rounding."""
    gh, gl, ga = got
    rh, rl, ra = ref
    rel = np.linalg.norm(gh - rh) / np.linalg.norm(rh)
    lmax = np.max(np.abs(gl - rl))
    print(f"{what}: hidden rel-L2 {rel:.3e} logits max-abs {lmax:.3e} argmax {ga} vs {ra}",
          flush=True)
    assert rel <= 1.5e-2
    assert lmax <= 5e-2
    assert rl[ga] >= rl.max() - 2 * 2.0**-8 * abs(rl.max())


def _tracks_plain_fp32(got, ref, ref32, what):
    """28 layers of bf16 activations: the GPU lands no further from the fp64 oracle than twice a
    plain fp32 implementation of the method does (evidence, not the fixed bar)."""
    gh, gl, ga = got
    rh, rl, ra = ref
    rel = np.linalg.norm(gh - rh) / np.linalg.norm(rh)
    lmax = np.max(np.abs(gl - rl))
    d32 = np.linalg.norm(ref32[0] - rh) / np.linalg.norm(rh)
    l32 = np.max(np.abs(ref32[1] - rl))
    print(f"{what}: hidden rel-L2 {rel:.3e} logits max-abs {lmax:.3e} argmax {ga} vs {ra} "
          f"(plain-fp32 oracle: {d32:.3e}, {l32:.3e})", flush=True)
    assert rel <= 2 * d32
    assert lmax <= 2 * l32
    assert rl[ga] >= rl.max() - 2 * 2.0**-8 * abs(rl.max()) - 2 * l32


def _check_kv(s, layer, n, oracle_model=None, min_equal=None):
    """The cache rows the prefill wrote against the oracle's (both bf16 values): relative L2 of
    K and of V within the fixed bar, and, when min_equal is given, at least that fraction of the
    elements bit-identical (layer 0, whose rows depend on the exact embedding rows only through
    roundings that rarely flip apart; later layers inherit the flips of the layers before)."""
    om = oracle_model or s.om
    kg, vg = s.kv_rows(layer, n)
    for got, ref in ((kg, om.k_cache[layer][:n]), (vg, om.v_cache[layer][:n])):
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        eq = float(np.mean(got == ref))
        print(f"  kv layer {layer}: rel-L2 {rel:.3e}, identical {eq:.5f}", flush=True)
        assert rel <= 1.5e-2, (layer, rel)
        if min_equal is not None:
            assert eq >= min_equal, (layer, eq)


@pytest.mark.timeout(600)
def test_prefill_two_layers_fixed_bar():
    """2 layers at the Qwen3-0.6B widths: a prefill of 100 tokens, a second of 37 at pos0 = 100
    (queries over cached keys), then a decode step at pos 137, each against the oracle decoding
    the same tokens one by one under the same 16-bit activation policy, at the fixed bar; the
    cache rows both prefills wrote against the oracle's."""
    s = PrefillSetup(SHAPE2)
    try:
        toks = synth.prompt_tokens(SHAPE["vocab"], 138, seed=4)
        got = s.prefill(toks[:100], 0)
        _, r64 = s.oracle_run(toks[:100], 0, fp32_pass=False)
        _fixed_bar(got, r64, "prefill 100")
        got = s.prefill(toks[100:137], 100)
        _, r64 = s.oracle_run(toks[100:137], 100, fp32_pass=False)
        _fixed_bar(got, r64, "prefill 37 at 100")
        for layer in range(2):
            _check_kv(s, layer, 137, min_equal=0.99 if layer == 0 else None)
        tok = torch.tensor([int(toks[137])], dtype=torch.int32, device=DEV)
        st = Q.make_step(137, token_id=tok, hidden_out=s.hidden, logits_out=s.logits,
                         argmax_out=s.amax)
        Q.qdec_decode_step(s.ctx, st)
        torch.cuda.synchronize()
        got = (s.hidden.cpu().numpy().astype(np.float64),
               synth.bf16_to_f32(s.logits).astype(np.float64), int(s.amax.item()))
        _, r64 = s.oracle_run(toks[137:], 137, fp32_pass=False)
        _fixed_bar(got, r64, "decode at 137")
        assert Q.qdec_device_error(s.ctx) == 0
    finally:
        s.close()


@pytest.mark.timeout(900)
def test_prefill_2048_tokens():
    """The benchmark's prefill: 2048 prompt tokens from position 0 in one call (every GEMM at
    m = 2048, the same launches the benchmark times).  At the Qwen3-0.6B widths with 2 layers:
    the last token's hidden state and logits at the fixed bar against the oracle decoding the
    2048 tokens one by one, and every K/V row the prefill wrote (2 layers x 2048 positions x 8
    heads) against the oracle's.  At the full 28 layers (the benchmark's model): the rows of
    layers 0 and 1 -- which depend only on the first two layers -- against the same oracle run,
    and the last token's greedy id valid for its own logits."""
    n = 2048
    toks = synth.prompt_tokens(SHAPE["vocab"], n, seed=4)
    s2 = PrefillSetup(SHAPE2, max_context=n, max_prefill=n)
    try:
        got = s2.prefill(toks, 0)
        print("prefill 2048 (2 layers) done; oracle decoding 2048 tokens", flush=True)
        _, r64 = s2.oracle_run(toks, 0, fp32_pass=False)
        _fixed_bar(got, r64, "prefill 2048, 2 layers")
        for layer in range(2):
            _check_kv(s2, layer, n, min_equal=0.99 if layer == 0 else None)
        om = s2.om
    finally:
        s2.close()
    s28 = PrefillSetup(SHAPE, max_context=n, max_prefill=n, oracle_model=False)
    try:
        gh, gl, ga = s28.prefill(toks, 0)
        print("prefill 2048 (28 layers) done", flush=True)
        assert np.all(np.isfinite(gh)) and np.all(np.isfinite(gl))
        assert gl[ga] == gl.max() and ga == int(np.flatnonzero(gl == gl.max())[0])
        for layer in range(2):
            _check_kv(s28, layer, n, oracle_model=om, min_equal=0.99 if layer == 0 else None)
        assert Q.qdec_device_error(s28.ctx) == 0
    finally:
        s28.close()


@pytest.mark.timeout(600)
def test_prefill_28_layers_track_plain_fp32():
    """The full 28 layers: a prefill of 100 tokens against the oracle decoding them one by one
    (evidence that the GPU lands where a plain fp32 implementation does after 28 layers of
    bf16 activations), and the cache rows of the first and last layer."""
    s = PrefillSetup()
    try:
        toks = synth.prompt_tokens(SHAPE["vocab"], 100, seed=4)
        got = s.prefill(toks, 0)
        r32, r64 = s.oracle_run(toks, 0)
        _tracks_plain_fp32(got, r64, r32, "prefill 100, 28 layers")
        _check_kv(s, 0, 100, min_equal=0.99)
        kg, vg = s.kv_rows(SHAPE["n_layers"] - 1, 100)
        for got_kv, ref in ((kg, s.om.k_cache[-1][:100]), (vg, s.om.v_cache[-1][:100])):
            assert np.linalg.norm(got_kv - ref) / np.linalg.norm(ref) <= 3e-2
    finally:
        s.close()


def test_prefill_rejects_bad_calls():
    s = PrefillSetup(max_context=256, max_prefill=32, oracle_model=False)
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
