"""The decode step at the 8B-class shape (36 layers, hidden 4096, 32 Q / 8 KV heads, D 128,
FFN 12288, vocab 151936 untied), bf16 weights or int4 weights with a scale per 128-value group
(the device quantises the same bf16 values the oracle's quantiser takes; codes are compared bit
for bit at op level), context 8192 with paged KV, all weights and KV resident in one GPU's HBM,
fp32 activations; one step at pos 8191 against the oracle with the fixed bar of the bf16 path
(hidden relative L2 <= 1.5e-2, logits max-abs <= 5e-2) and the tighter bar of the Qwen3-shape
test: hidden relative L2 <= max(1e-4, 4 d32), every logit within one bf16 spacing
(2^-7 |logit| plus 1e-5 of the largest) plus 4 l32, where d32 / l32 are the plain-fp32 oracle
mode's distances from the fp64 result; greedy id a maximiser of the oracle's logits up to bf16
rounding."""
import numpy as np
import pytest
import torch

import oracle
from decode_step_04_amd import loader, synth
from decode_step_04_amd import qdec as Q

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPE = synth.DENSE_8B
T = 8192


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", ["bf16", "w4a16"])
def test_8b_step_matches_oracle(path):
    print(f"8b setup path={path}", flush=True)
    n_pages = T // 16
    cfg = loader.config_for(SHAPE, path=path, num_pages=n_pages, max_context=T)
    ctx = Q.qdec_create(cfg, 0)
    try:
        w = synth.bf16_model(SHAPE, seed=0, device=DEV)
        loader.upload_weights(ctx, w, DEV)
        table = synth.block_table(n_pages, n_pages, seed=2)
        Q.qdec_kv_set_block_table(ctx, table)
        kv = synth.kv_prefill(SHAPE, T - 1, seed=1, device=DEV)
        loader.prefill_kv(ctx, kv)
        tok_id = synth.token_id(SHAPE["vocab"], seed=3)
        tok = torch.tensor([tok_id], dtype=torch.int32, device=DEV)
        hidden = torch.empty(SHAPE["hidden"], device=DEV)
        logits = torch.empty(SHAPE["vocab"], dtype=torch.bfloat16, device=DEV)
        amax = torch.empty(1, dtype=torch.int32, device=DEV)
        Q.qdec_decode_step(ctx, Q.make_step(T - 1, token_id=tok, hidden_out=hidden,
                                            logits_out=logits, argmax_out=amax))
        torch.cuda.synchronize()
        gh = hidden.cpu().numpy().astype(np.float64)
        gl = synth.bf16_to_f32(logits).astype(np.float64)
        ga = int(amax.item())
        print("8b oracle", flush=True)
        hw = synth.host_weights(w)
        del w
        if path == "w4a16":
            for key in ("qkv", "o", "gate_up", "down"):
                qs = [oracle.quantize_groups(oracle.bf16_bits_to_f64(b).astype(np.float32), 4)
                      for b in hw[key]]
                hw[key] = [q for q, _ in qs]
                hw[key + "_scale"] = [s for _, s in qs]
            q, s = oracle.quantize_groups(oracle.bf16_bits_to_f64(hw["lm_head"]).astype(np.float32), 4)
            hw["lm_head"], hw["lm_scale"] = q, s
        om = oracle.Model(dict(SHAPE, act_bf16=0, kv_bf16=1, logits_bf16=1), hw, max_ctx=T)
        for l, (k, v) in enumerate(kv):
            om.k_cache[l][: T - 1] = k.float().cpu().numpy()
            om.v_cache[l][: T - 1] = v.float().cpu().numpy()
        del kv
        with oracle.fp32_arithmetic():
            r32 = om.step(T - 1, token=tok_id)
        rh, rl, ra = om.step(T - 1, token=tok_id)
        rel = np.linalg.norm(gh - rh) / np.linalg.norm(rh)
        lmax = np.max(np.abs(gl - rl))
        d32 = np.linalg.norm(r32[0] - rh) / np.linalg.norm(rh)
        l32 = np.max(np.abs(r32[1] - rl))
        print(f"8b {path} hidden rel-L2 {rel:.3e} logits max-abs {lmax:.3e} argmax {ga} vs {ra} "
              f"(plain-fp32 oracle: {d32:.3e}, {l32:.3e})", flush=True)
        assert rel <= 1.5e-2 and lmax <= 5e-2
        assert rel <= max(1e-4, 4 * d32)
        assert np.all(np.abs(gl - rl) <= 2.0**-7 * np.abs(rl) + 1e-5 * np.abs(rl).max() + 4 * l32)
        assert rl[ga] >= rl.max() - 2 * 2.0**-8 * abs(rl.max())
    finally:
        Q.qdec_destroy(ctx)
