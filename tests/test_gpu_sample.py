"""Device-side temperature + top-p sampling (through the C ABI) against the oracle.

The oracle draws u from its own Philox4x32-10 and samples by definition in fp64; the device uses
fp32 exponentials and exact fixed-point sums.  Where the two could differ -- a draw or the nucleus
boundary within a hair of a cumulative step -- several tokens are correct, so the device's token
must be one the oracle returns when u and top_p move by at most DELTA; almost every draw must
match exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_step_04_amd import qdec as Q
from decode_step_04_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
DELTA = 1e-5


def _ws(n):
    return torch.empty(Q.qdec_op_sample_workspace(n), dtype=torch.uint8, device=DEV)


def _sample(logits, dt, n, temp, top_p, seed, pos, ws, out):
    Q.qdec_op_sample(logits, dt, n, temp, top_p, seed, pos, ws, ws.numel(), out)


def _allowed(z, temp, top_p, u):
    out = set()
    for tp in (top_p - DELTA, top_p, min(1.0, top_p + DELTA)):
        for uu in (max(0.0, u - DELTA), u, min(1.0 - 1e-12, u + DELTA)):
            out.add(oracle.sample(z, temp, max(tp, 1e-12), uu)[0])
    return out


@pytest.mark.parametrize("n,dt", [(10, "f32"), (1000, "bf16"), (4096, "f32"), (151936, "bf16")])
@pytest.mark.parametrize("temp,top_p", [(1.0, 1.0), (0.7, 0.9), (1.5, 0.5), (0.3, 0.05)])
def test_sample_matches_oracle(n, dt, temp, top_p):
    print(f"sample n={n} dt={dt} T={temp} top_p={top_p}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(n + int(temp * 10) + int(top_p * 100))
    logits = torch.randn(n, generator=g, device=DEV) * 3.0
    if dt == "bf16":
        logits = logits.to(torch.bfloat16)
        z = synth.bf16_to_f32(logits).astype(np.float64)
    else:
        z = logits.cpu().numpy().astype(np.float64)
    draws = 40 if n <= 4096 else 12
    seed = 0x1234_5678_9ABC_DEF0 + n
    out = torch.empty(draws, dtype=torch.int32, device=DEV)
    ws = _ws(n)
    for pos in range(draws):
        _sample(logits, Q.BF16 if dt == "bf16" else Q.F32, n, temp, top_p, seed, pos, ws,
                out[pos:])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    exact = 0
    for pos in range(draws):
        u = oracle.sample_uniform(seed, pos)
        want = oracle.sample(z, temp, top_p, u)[0]
        exact += int(got[pos] == want)
        assert got[pos] in _allowed(z, temp, top_p, u), (pos, int(got[pos]), want)
    assert exact >= draws - 1


def test_sample_ties_and_greedy_limit():
    n = 64
    flat = torch.zeros(n, device=DEV)                  # all equal: the nucleus is by index
    out = torch.empty(200, dtype=torch.int32, device=DEV)
    ws = _ws(5000)
    for pos in range(200):
        _sample(flat, Q.F32, n, 1.0, 0.1, 99, pos, ws, out[pos:])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # 0.1 of 64 equal tokens: the first 7 (mass 7/64 >= 0.1)
    assert set(got.tolist()) == set(range(7))
    peaked = torch.randn(5000, generator=torch.Generator(device=DEV).manual_seed(2), device=DEV)
    am = int(torch.argmax(peaked).item())
    _sample(peaked, Q.F32, 5000, 1.0, 1e-6, 7, 3, ws, out)
    _sample(peaked, Q.F32, 5000, 1e-3, 0.99, 7, 4, ws, out[1:])
    torch.cuda.synchronize()
    assert out[0].item() == am and out[1].item() == am


@pytest.mark.parametrize("case", ["flat_f32", "levels_f32", "levels_bf16"])
def test_sample_many_candidates(case):
    """2^18 logits whose boundary bin holds more candidates than the selection work-group keeps
    in LDS (the candidates are then read from the workspace), with wide exact ties.  The logits
    sit on a coarse grid so that equal logits are the only equal probabilities on both sides."""
    n = 1 << 18
    print(f"sample many candidates {case}", flush=True)
    rng = np.random.default_rng(5)
    if case == "flat_f32":
        z = np.zeros(n)
    elif case == "levels_f32":
        z = np.round(rng.standard_normal(n) * 12.0) / 64.0
    else:
        z = synth.bf16_to_f32(torch.from_numpy(rng.standard_normal(n) * 0.05 + 1.0).float()
                              .to(torch.bfloat16)).astype(np.float64)
    dt = Q.BF16 if case.endswith("bf16") else Q.F32
    logits = torch.from_numpy(z).float().to(DEV)
    if dt == Q.BF16:
        logits = logits.to(torch.bfloat16)
    ws = _ws(n)
    out = torch.empty(8, dtype=torch.int32, device=DEV)
    seed = 77
    for pos, (temp, top_p) in enumerate([(1.0, 0.5), (1.0, 0.95), (0.5, 0.3), (2.0, 0.999),
                                         (1.0, 1.0), (0.25, 0.7), (1.0, 0.05), (3.0, 0.6)]):
        _sample(logits, dt, n, temp, top_p, seed, pos, ws, out[pos:])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for pos, (temp, top_p) in enumerate([(1.0, 0.5), (1.0, 0.95), (0.5, 0.3), (2.0, 0.999),
                                         (1.0, 1.0), (0.25, 0.7), (1.0, 0.05), (3.0, 0.6)]):
        u = oracle.sample_uniform(seed, pos)
        assert got[pos] in _allowed(z, temp, top_p, u), (case, pos, int(got[pos]))


def test_sample_small_rows_and_nan():
    """Rows shorter than the number of slices, and NaN logits, which are never drawn (the
    oracle sees them as -inf)."""
    ws = _ws(1 << 18)
    out = torch.empty(1, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(6)
    for n in (1, 2, 3, 63, 65, 257):
        z = rng.standard_normal(n) * 2.0
        lg = torch.from_numpy(z).float().to(DEV)
        for pos in range(6):
            _sample(lg, Q.F32, n, 1.0, 0.8, 5, pos, ws, out)
            torch.cuda.synchronize()
            assert int(out.item()) in _allowed(z, 1.0, 0.8, oracle.sample_uniform(5, pos)), (n, pos)
    z = rng.standard_normal(3000) * 2.0
    z[::7] = np.nan
    lg = torch.from_numpy(z).float().to(DEV)
    zo = np.where(np.isnan(z), -np.inf, z)
    for pos in range(12):
        _sample(lg, Q.F32, 3000, 1.0, 0.99, 8, pos, ws, out)
        torch.cuda.synchronize()
        t = int(out.item())
        assert t % 7 != 0 and t in _allowed(zo, 1.0, 0.99, oracle.sample_uniform(8, pos))


def test_sample_rejects_bad_arguments():
    x = torch.zeros(16, device=DEV)
    out = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = _ws(16)
    for temp, top_p, pos in ((0.0, 0.9, 0), (1.0, 0.0, 0), (1.0, 1.5, 0), (1.0, 0.9, -1)):
        with pytest.raises(Q.QdecError):
            _sample(x, Q.F32, 16, temp, top_p, 1, pos, ws, out)
    with pytest.raises(Q.QdecError):  # workspace too small
        Q.qdec_op_sample(x, Q.F32, 16, 1.0, 0.9, 1, 0, ws, ws.numel() - 1, out)
    with pytest.raises(Q.QdecError):
        Q.qdec_op_sample_workspace((1 << 18) + 1)


def test_decode_step_samples_and_graph_replays_match():
    """The tiny fp32 decoder decoding with temperature 0.8 / top_p 0.9: every sampled id is one
    the oracle's sampler gives on the step's own logits with the step's Philox draw (up to
    DELTA), the id feeds the next step on the device, and a graph replay of the same sampling
    step reproduces the eager ids."""
    from decode_step_04_amd import loader

    m = synth.tiny_model(seed=0)
    cfg = m["cfg"]

    def run(use_graph):
        c = loader.config_for(cfg, path="fp32", num_pages=m["num_pages"], max_context=64)
        ctx = Q.qdec_create(c, 0)
        try:
            loader.upload_weights(ctx, m["weights"], DEV)
            Q.qdec_kv_set_block_table(ctx, m["block_table"])
            tok = torch.tensor([int(m["prompt"][0])], dtype=torch.int32, device=DEV)
            lg = torch.zeros(cfg["vocab"], device=DEV)
            st = Q.make_step(0, token_id=tok, logits_out=lg, argmax_out=tok, temperature=0.8,
                             top_p=0.9, seed=2024)
            if use_graph:
                Q.qdec_graph_capture(ctx, st)
            ids, logs = [], []
            for pos in range(24):
                if use_graph:
                    Q.qdec_graph_replay(ctx, pos)
                else:
                    st.pos = pos
                    Q.qdec_decode_step(ctx, st)
                torch.cuda.synchronize()
                ids.append(int(tok.item()))
                logs.append(lg.cpu().numpy().astype(np.float64))
            return ids, logs
        finally:
            Q.qdec_destroy(ctx)

    ids, logs = run(False)
    for pos, (t, z) in enumerate(zip(ids, logs)):
        u = oracle.sample_uniform(2024, pos)
        assert t in _allowed(z, 0.8, 0.9, u), (pos, t)
    ids_g, _ = run(True)
    assert ids_g == ids
    assert len(set(ids)) > 3          # it is sampling, not repeating one greedy id
