"""Helpers that marshal a model's tensors into a qdec context (no arithmetic of the method).

``config_for`` fills a ``qdec_config`` from a shape dict (see ``synth``); ``upload_weights``
hands every tensor of a weight dict to ``qdec_upload`` (the library converts / quantises on the
device); ``prefill_kv`` writes logical K/V rows through the block table with ``qdec_kv_write``.
"""
from __future__ import annotations

from . import qdec as Q


# quantised paths: weight storage type of the projections and the LM head
QUANT_PATHS = {"w8a16": Q.I8_ROW, "w8a16g": Q.I8_G128, "w4a16": Q.I4_G128}
# bf16 layers with an int8 per-row LM head only: the shipped mode of the Qwen3 runtime page
# (its W8A16 section quantises the LM head alone)
LM_ONLY_PATHS = {"bf16-w8head": Q.I8_ROW}


def config_for(shape: dict, *, path: str, num_pages: int, max_context: int,
               partition_size: int = 0, act: str = None, max_prefill: int = 0,
               weight_slots: int = 0) -> Q.qdec_config:
    """path: 'fp32' (fp32 everything), 'bf16' (bf16 weights, embedding, logits and KV), 'w8a16'
    (int8 per-row projections and LM head, bf16 embedding, logits and KV), 'w8a16g' (int8 with a
    scale per 128-value group), 'w4a16' (int4 with a scale per 128-value group) or 'bf16-w8head'
    (bf16 projections, int8 per-row LM head, bf16 embedding, logits and KV).  act: 'f32' or 'bf16',
    the precision of activations crossing op boundaries; default 'f32' for every path (the weight
    and cache formats are storage formats; activations are a few KiB per step, so their precision
    costs no bandwidth), 'bf16' rounds them to 16 bits at every op boundary.  weight_slots: 0 keeps
    every layer's projections in device memory; N >= 1 streams them from pinned host memory
    through N device slots."""
    if path == "fp32":
        proj = lm = io = kv = Q.F32
        act = act or "f32"
    elif path == "bf16":
        proj = lm = io = kv = Q.BF16
        act = act or "f32"
    elif path in QUANT_PATHS:
        proj = lm = QUANT_PATHS[path]
        io = kv = Q.BF16
        act = act or "f32"
    elif path in LM_ONLY_PATHS:
        proj = io = kv = Q.BF16
        lm = LM_ONLY_PATHS[path]
        act = act or "f32"
    else:
        raise ValueError(path)
    act = Q.F32 if act == "f32" else Q.BF16
    return Q.make_config(
        n_layers=shape["n_layers"], hidden=shape["hidden"], n_q_heads=shape["n_q_heads"],
        n_kv_heads=shape["n_kv_heads"], head_dim=shape["head_dim"], ffn=shape["ffn"],
        vocab=shape["vocab"], tied_lm_head=int(shape["tied"]), qk_norm=int(shape["qk_norm"]),
        rms_eps=shape["eps"], rope_theta=shape["theta"], proj_dtype=proj, lm_head_dtype=lm,
        io_dtype=io, act_dtype=act, kv_dtype=kv, page_size=16, num_pages=num_pages, max_context=max_context,
        partition_size=partition_size, max_prefill=max_prefill, weight_slots=weight_slots)


def _dt(t):
    import torch

    if t.dtype == torch.float32:
        return Q.F32
    if t.dtype == torch.bfloat16:
        return Q.BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def upload_weights(ctx, weights: dict, device="cuda", stream=None):
    """Uploads a weight dict (torch tensors, or numpy float32 arrays for the tiny model).
    Tensors are moved to `device` first so every conversion runs on the GPU."""
    import numpy as np
    import torch

    keep = []

    def dev(a):
        if isinstance(a, np.ndarray):
            a = torch.from_numpy(a)
        t = a.to(device).contiguous()
        keep.append(t)
        return t

    def up(layer, which, a):
        t = dev(a)
        rows, cols = (1, t.numel()) if t.dim() == 1 else tuple(t.shape)
        Q.qdec_upload(ctx, layer, which, t, _dt(t), rows, cols, 1, stream)

    up(0, Q.W_EMBED, weights["embed"])
    if weights.get("lm_head") is not None:
        up(0, Q.W_LM_HEAD, weights["lm_head"])
    up(0, Q.W_FINAL_NORM, weights["final_norm"])
    for l in range(len(weights["qkv"])):
        up(l, Q.W_IN_NORM, weights["in_norm"][l])
        up(l, Q.W_POST_NORM, weights["post_norm"][l])
        if weights.get("q_norm"):
            up(l, Q.W_Q_NORM, weights["q_norm"][l])
            up(l, Q.W_K_NORM, weights["k_norm"][l])
        up(l, Q.W_QKV, weights["qkv"][l])
        up(l, Q.W_O, weights["o"][l])
        up(l, Q.W_GATE_UP, weights["gate_up"][l])
        up(l, Q.W_DOWN, weights["down"][l])
    torch.cuda.synchronize()
    del keep


def prefill_kv(ctx, kv_layers, stream=None):
    """kv_layers: list over layers of (K, V) device tensors [n, Hkv, D] in the KV dtype,
    written at positions 0..n-1."""
    for l, (k, v) in enumerate(kv_layers):
        Q.qdec_kv_write(ctx, l, 0, k.shape[0], k.contiguous(), v.contiguous(), stream)
