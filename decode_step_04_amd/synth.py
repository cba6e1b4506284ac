"""Seeded synthetic inputs for the decode step (weights, KV pre-fill, block tables, queries).

This module holds no arithmetic of the method (no norm, projection, rotation, attention or
quantisation): it only draws random numbers and stores them in the storage types the workloads
name.  Both the HIP path's tests and the oracle's tests take their inputs from here.

Workloads (shapes from the Qwen3 runtime page, §1.1, and the benchmark configurations):
  tiny   fp32 GQA decoder: 2 layers, hidden 256, 4 Q / 2 KV heads, D 64, FFN 768, vocab 512 tied
  0.6b   Qwen3-0.6B shape: 28 layers, hidden 1024, 16 Q / 8 KV heads, D 128, FFN 3072, vocab
         151936 tied
  8b     8B-class shape: 36 layers, hidden 4096, 32 Q / 8 KV heads, D 128, FFN 12288, vocab 151936
         untied
Value distributions: matrices N(0, 0.02), norm gammas 1 + N(0, 0.1), pre-filled K/V N(0, 1),
token ids uniform, block tables uniform random permutations of the physical pages.
"""
from __future__ import annotations

import numpy as np

TINY = dict(name="tiny-fp32", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
            ffn=768, vocab=512, tied=1, qk_norm=1, eps=1e-6, theta=1e6)
QWEN3_0P6B = dict(name="qwen3-0.6b-shape", n_layers=28, hidden=1024, n_q_heads=16, n_kv_heads=8,
                  head_dim=128, ffn=3072, vocab=151936, tied=1, qk_norm=1, eps=1e-6, theta=1e6)
DENSE_8B = dict(name="8b-class-shape", n_layers=36, hidden=4096, n_q_heads=32, n_kv_heads=8,
                head_dim=128, ffn=12288, vocab=151936, tied=0, qk_norm=1, eps=1e-6, theta=1e6)
PAGE = 16


def matrix_shapes(cfg: dict) -> dict:
    """Row-major [out x in] shapes of one layer's matrices and the global tables."""
    d, hq, hkv, hd, f, v = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                             "ffn", "vocab"))
    return dict(qkv=((hq + 2 * hkv) * hd, d), o=(d, hq * hd), gate_up=(2 * f, d), down=(d, f),
                embed=(v, d))


# ---- tiny fp32 model (numpy, host) ------------------------------------------------------------

def tiny_model(seed: int = 0, prompt_len: int = 16, num_pages: int = 8) -> dict:
    """Weights, prompt and block table of the tiny fp32 decoder.

    numpy ``default_rng(seed)`` draws, in this order: embedding [V, d]; per layer: input gamma,
    QKV, Q gamma, K gamma, O, post-attention gamma, gate-up, down; final gamma; the prompt's
    token ids; the block-table permutation.
    """
    cfg = TINY
    rng = np.random.default_rng(seed)
    sh = matrix_shapes(cfg)
    d, hd = cfg["hidden"], cfg["head_dim"]

    def mat(shape):
        return (rng.standard_normal(shape) * 0.02).astype(np.float32)

    def gamma(n):
        return (1.0 + rng.standard_normal(n) * 0.1).astype(np.float32)

    w = dict(embed=mat(sh["embed"]), lm_head=None, qkv=[], o=[], gate_up=[], down=[],
             in_norm=[], post_norm=[], q_norm=[], k_norm=[])
    for _ in range(cfg["n_layers"]):
        w["in_norm"].append(gamma(d))
        w["qkv"].append(mat(sh["qkv"]))
        w["q_norm"].append(gamma(hd))
        w["k_norm"].append(gamma(hd))
        w["o"].append(mat(sh["o"]))
        w["post_norm"].append(gamma(d))
        w["gate_up"].append(mat(sh["gate_up"]))
        w["down"].append(mat(sh["down"]))
    w["final_norm"] = gamma(d)
    prompt = rng.integers(0, cfg["vocab"], size=prompt_len).astype(np.int32)
    table = rng.permutation(num_pages).astype(np.int32)
    return dict(cfg=cfg, weights=w, prompt=prompt, block_table=table, num_pages=num_pages)


# ---- bf16 models (torch, any device) -------------------------------------------------------------

def bf16_model(cfg: dict, seed: int = 0, device="cpu"):
    """Weights of a bf16 model drawn with a torch generator on `device`.

    Matrices are drawn in fp32 as N(0, 0.02) and stored as bf16 (torch's round-to-nearest-even
    cast); gammas are fp32 1 + N(0, 0.1).  Order: embedding, per layer (input gamma, QKV, Q gamma,
    K gamma, O, post gamma, gate-up, down), final gamma, then the untied LM head if any.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    sh = matrix_shapes(cfg)
    d, hd = cfg["hidden"], cfg["head_dim"]

    def mat(shape):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32)
                .mul_(0.02).to(torch.bfloat16))

    def gamma(n):
        return torch.randn(n, generator=g, device=device, dtype=torch.float32).mul_(0.1).add_(1.0)

    w = dict(embed=mat(sh["embed"]), qkv=[], o=[], gate_up=[], down=[], in_norm=[],
             post_norm=[], q_norm=[], k_norm=[])
    for _ in range(cfg["n_layers"]):
        w["in_norm"].append(gamma(d))
        w["qkv"].append(mat(sh["qkv"]))
        w["q_norm"].append(gamma(hd))
        w["k_norm"].append(gamma(hd))
        w["o"].append(mat(sh["o"]))
        w["post_norm"].append(gamma(d))
        w["gate_up"].append(mat(sh["gate_up"]))
        w["down"].append(mat(sh["down"]))
    w["final_norm"] = gamma(d)
    w["lm_head"] = None if cfg["tied"] else mat(sh["embed"])
    return w


def kv_prefill(cfg: dict, n_pos: int, seed: int = 1, device="cpu"):
    """Per-layer logical K and V [n_pos, Hkv, D] bf16, N(0, 1), for positions 0..n_pos-1."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (n_pos, cfg["n_kv_heads"], cfg["head_dim"])
    out = []
    for _ in range(cfg["n_layers"]):
        k = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        v = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        out.append((k, v))
    return out


def block_table(num_pages: int, n_logical: int, seed: int = 2) -> np.ndarray:
    """First n_logical entries of a uniform random permutation of the physical pages."""
    rng = np.random.default_rng(seed)
    return rng.permutation(num_pages)[:n_logical].astype(np.int32)


def token_id(vocab: int, seed: int = 3) -> int:
    return int(np.random.default_rng(seed).integers(0, vocab))


def prompt_tokens(vocab: int, n: int, seed: int = 4) -> np.ndarray:
    """n token ids, uniform in [0, vocab) (a synthetic prompt for prefill)."""
    return np.random.default_rng(seed).integers(0, vocab, size=n).astype(np.int32)


# ---- attention stress (one layer, 32 Q / 8 KV heads, D 128) ---------------------------------------

STRESS = dict(n_q_heads=32, n_kv_heads=8, head_dim=128)


def attention_stress(ctx: int, seed: int = 4, device="cpu", score_span: float = 20.0):
    """q fp32 [32, 128]; K, V bf16 [ctx, 8, 128] ~ N(0, 1); a block table over exactly the
    needed pages.  Each q head is drawn N(0, 1) and rescaled to norm
    sqrt(D) * score_span / sqrt(2 ln ctx): with unit-variance keys the scaled scores then have
    standard deviation score_span / sqrt(2 ln ctx), so the largest of ctx of them is close to
    +-score_span (the expected maximum of n standard normals is about sqrt(2 ln n)).
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    hq, hkv, d = STRESS["n_q_heads"], STRESS["n_kv_heads"], STRESS["head_dim"]
    q = torch.randn((hq, d), generator=g, device=device, dtype=torch.float64)
    target = np.sqrt(d) * score_span / np.sqrt(2.0 * np.log(max(ctx, 2)))
    q = (q / q.norm(dim=1, keepdim=True) * target).to(torch.float32)
    k = torch.randn((ctx, hkv, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((ctx, hkv, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    n_pages = (ctx + PAGE - 1) // PAGE
    table = block_table(n_pages, n_pages, seed=seed + 100)
    return q, k, v, table


# ---- W8A16 GEMV ---------------------------------------------------------------------------------

GEMV_SHAPES = ((130560, 1536), (151936, 1024))


def gemv_inputs(n: int, k: int, seed: int = 5, device="cpu"):
    """W fp32 [n, k] ~ N(0, 0.02) (quantised per row by the code under test) and x bf16 [k] ~ N(0, 1)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32).mul_(0.02)
    x = torch.randn((k,), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return w, x


# ---- conversions between torch storage and the numpy arrays the oracle reads -----------------------

def bf16_to_bits(t) -> np.ndarray:
    """torch bf16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f32(t) -> np.ndarray:
    """torch bf16 tensor -> numpy float32 array of the same values (exact)."""
    import torch

    return t.detach().to(torch.float32).cpu().numpy()


def host_weights(w: dict) -> dict:
    """Host copy of a weight dict for the oracle: bf16 tensors become uint16 bit arrays, fp32
    tensors float32 arrays, lists stay lists."""
    import torch

    def h(t):
        if t is None:
            return None
        if isinstance(t, np.ndarray):
            return t
        return bf16_to_bits(t) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()

    return {k: ([h(t) for t in v] if isinstance(v, list) else h(v)) for k, v in w.items()}
