"""The split-KV merge of the decode step, through the C ABI, against the oracle.

The attention kernel writes each partition's (m, l, acc) state; the merge kernel folds them: with
at most 32 partitions per head in one chunk by one wave, with more in chunks of 32 dealt to four
waves and combined through LDS.  Both are the exact merge of the page "从 Qwen3 数学到 CUDA
Kernel：0.6B 推理运行时的完整实现与优化" (§9.1, §10.1).

Recipe: the tiny fp32 decoder (seed 0: 2 layers, hidden 256, 4 Q / 2 KV heads, D 64, FFN 768,
vocab 512), partitions of 64 tokens, max_context 2048 (32 partitions: one chunk) or 4096 (64
partitions: four waves), every KV position pre-filled with N(0, 1) values (seed 1) through a
random permutation of the pool pages (seed 2), one token id (seed 3); decode steps at a sequence
of positions that mixes one, two, a few and all partitions, in the same order on the GPU and in
the oracle (each step appends its own K/V row, which later steps read).  Bar: hidden state and
logits within max-abs 1e-4 of the fp64 oracle (the fp32 path's bar); graph replays (grid over
every partition of max_context: surplus work-groups store nothing, the merge reads only the
step's partitions) bit-identical to the eager steps, over two rounds of the sequence.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_step_04_amd import loader, synth
from decode_step_04_amd import qdec as Q

pytestmark = pytest.mark.gpu
DEV = "cuda"
PART = 64


def positions(max_ctx):
    return (max_ctx - 1, 0, 63, 64, 700, 129, max_ctx - 1, 1000)


class Setup:
    def __init__(self, max_ctx):
        print(f"step merge setup max_context={max_ctx} partition={PART}", flush=True)
        self.m = synth.tiny_model(seed=0)
        self.cfgd = self.m["cfg"]
        self.max_ctx = max_ctx
        n_pages = max_ctx // 16
        self.c = loader.config_for(self.cfgd, path="fp32", num_pages=n_pages, max_context=max_ctx,
                                   partition_size=PART)
        self.ctx = Q.qdec_create(self.c, 0)
        loader.upload_weights(self.ctx, self.m["weights"], DEV)
        Q.qdec_kv_set_block_table(self.ctx, synth.block_table(n_pages, n_pages, seed=2))
        self.kv = [(k.float(), v.float())
                   for k, v in synth.kv_prefill(self.cfgd, max_ctx, seed=1, device=DEV)]
        self.tok_id = synth.token_id(self.cfgd["vocab"], seed=3)
        self.tok = torch.tensor([self.tok_id], dtype=torch.int32, device=DEV)
        self.hid = torch.zeros(self.cfgd["hidden"], device=DEV)
        self.lg = torch.zeros(self.cfgd["vocab"], device=DEV)
        self.info = Q.qdec_info_get(self.ctx)

    def close(self):
        Q.qdec_destroy(self.ctx)

    def run(self, pos_seq, graph):
        loader.prefill_kv(self.ctx, self.kv)
        torch.cuda.synchronize()
        st = Q.make_step(0, token_id=self.tok, hidden_out=self.hid, logits_out=self.lg)
        if graph:
            Q.qdec_graph_capture(self.ctx, st)
        out = []
        for p in pos_seq:
            print(f"  step pos={p} graph={graph}", flush=True)
            self.tok.fill_(self.tok_id)
            if graph:
                Q.qdec_graph_replay(self.ctx, p)
            else:
                st.pos = p
                Q.qdec_decode_step(self.ctx, st)
            torch.cuda.synchronize()
            out.append((self.hid.cpu().numpy().copy(), self.lg.cpu().numpy().copy()))
        return out

    def oracle_run(self, pos_seq):
        om = oracle.Model(dict(self.cfgd, act_bf16=0, kv_bf16=0), self.m["weights"],
                          max_ctx=self.max_ctx)
        for l, (k, v) in enumerate(self.kv):
            om.k_cache[l][:] = k.cpu().numpy()
            om.v_cache[l][:] = v.cpu().numpy()
        out = []
        for p in pos_seq:
            h, lg, _ = om.step(p, token=self.tok_id, want_logits=True)
            out.append((h, lg))
        return out


@pytest.mark.parametrize("max_ctx", [2048, 4096])
def test_merge_matches_oracle_and_graph_replays(max_ctx):
    s = Setup(max_ctx)
    try:
        assert s.info.max_partitions == max_ctx // PART
        seq = positions(max_ctx)
        ref = s.oracle_run(seq)
        eager = s.run(seq, graph=False)
        for p, (h, lg), (rh, rl) in zip(seq, eager, ref):
            dh, dl = np.max(np.abs(h - rh)), np.max(np.abs(lg - rl))
            print(f"pos {p}: hidden max-abs {dh:.2e} logits max-abs {dl:.2e}", flush=True)
            assert dh <= 1e-4 and dl <= 1e-4, p
        for _ in range(2):
            replay = s.run(seq, graph=True)
            for p, (h, lg), (eh, el) in zip(seq, replay, eager):
                assert np.array_equal(h, eh) and np.array_equal(lg, el), p
    finally:
        s.close()
