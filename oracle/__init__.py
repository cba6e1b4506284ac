"""CPU oracle for the batch-1 GQA decode step (test infrastructure only).

Thin ctypes wrapper around ``liboracle.so`` (built from ``oracle.c`` by ``oracle/build.py``).
Only the tests, the smoke check and the benchmark's CPU-baseline leg import this package; the
HIP library and its Python binding never do.  Arrays go in and come out as numpy arrays; all
floating-point results are float64.  See ``oracle.c`` for what each function computes and which
passage of the pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OR_F32, OR_BF16, OR_I8, OR_I8G, OR_I4G = 0, 1, 2, 3, 4
GROUP = 128  # values per scale in the group-wise formats

_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_D = C.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b  # noqa: F401  (build script lives beside the source)
            _b.build()
        _lib = C.CDLL(_LIB_PATH)
        sig = {
            "or_round_bf16": (None, [_P, _P, _I64]),
            "or_to_bf16_bits": (None, [_P, _P, _I64]),
            "or_bf16_bits_to_double": (None, [_P, _P, _I64]),
            "or_params_per_layer": (_I64, [_I64, _I64, _I64, _I64, _I64, _I32]),
            "or_params_total": (_I64, [_I64] * 7 + [_I32, _I32]),
            "or_kv_bytes_per_layer_token": (_I64, [_I64, _I64, _I64]),
            "or_rmsnorm": (None, [_P, _P, _I64, _D, _P]),
            "or_silu": (None, [_P, _P, _I64]),
            "or_rope": (None, [_P, _I32, _I64, _D]),
            "or_gemv": (None, [_P, _I32, _P, _P, _I64, _I64, _P]),
            "or_quantize_rows": (None, [_P, _I64, _I64, _P, _P]),
            "or_quantize_groups": (None, [_P, _I64, _I64, _I32, _P, _P]),
            "or_attention": (None, [_P, _P, _P, _I64, _I32, _I32, _I32, _P]),
            "or_attention_online": (None, [_P, _P, _P, _I64, _I32, _I32, _I32, _P]),
            "or_attention_partitioned": (None, [_P, _P, _P, _I64, _I32, _I32, _I32, _I64, _P]),
            "or_pool_offset": (_I64, [_I32, _I32, _I32, _P, _I32, _I32, _I32]),
            "or_pool_scatter": (None, [_P, _I32, _I32, _I32, _P, _I32, _I32, _I32, _P]),
            "or_decode_step": (_I32, [_P, _I32, _P, _I32, _P, _P, _P]),
            "or_argmax": (_I64, [_P, _I64]),
            "or_set_fp32": (None, [_I32]),
            "or_philox4x32_10": (None, [_P, _P, _P]),
            "or_sample_uniform": (_D, [C.c_uint64, _I64]),
            "or_sample": (_I64, [_P, _I64, _D, _D, _D, _P, _P]),
            "or_get_fp32": (_I32, []),
            "or_set_threads": (None, [_I32]),
            "or_get_threads": (_I32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(_lib, name)
            fn.restype = res
            fn.argtypes = args
    return _lib


def set_threads(n: int) -> None:
    """Threads the OpenMP loops use (timing only; results do not depend on it)."""
    lib().or_set_threads(int(n))


def get_threads() -> int:
    return int(lib().or_get_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class fp32_arithmetic:
    """Context manager: inside it every oracle function computes in plain sequential fp32 (each
    partial sum, unfused product and function value rounded to fp32) instead of fp64.  Used only
    to measure a plain fp32 implementation's distance from the fp64 result; the parity
    reference is always the default fp64 mode."""

    def __enter__(self):
        self._prev = lib().or_get_fp32()
        lib().or_set_fp32(1)
        return self

    def __exit__(self, *exc):
        lib().or_set_fp32(self._prev)
        return False


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---- number formats ------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    lib().or_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def to_bf16_bits(x) -> np.ndarray:
    x = _f64(x)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().or_to_bf16_bits(_ptr(x), _ptr(out), x.size)
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().or_bf16_bits_to_double(_ptr(bits), _ptr(out), bits.size)
    return out


# ---- shapes ---------------------------------------------------------------------------------

def params_per_layer(hidden, hq, hkv, d, ffn, qk_norm=1) -> int:
    return int(lib().or_params_per_layer(hidden, hq, hkv, d, ffn, qk_norm))


def params_total(n_layers, hidden, hq, hkv, d, ffn, vocab, tied, qk_norm=1) -> int:
    return int(lib().or_params_total(n_layers, hidden, hq, hkv, d, ffn, vocab, tied, qk_norm))


def kv_bytes_per_layer_token(hkv, d, elem) -> int:
    return int(lib().or_kv_bytes_per_layer_token(hkv, d, elem))


# ---- ops -------------------------------------------------------------------------------------

def rmsnorm(x, gamma, eps) -> np.ndarray:
    x = _f64(x)
    g = _f32(gamma)
    out = np.empty_like(x)
    lib().or_rmsnorm(_ptr(x), _ptr(g), x.size, float(eps), _ptr(out))
    return out


def silu(z) -> np.ndarray:
    z = _f64(z)
    out = np.empty_like(z)
    lib().or_silu(_ptr(z), _ptr(out), z.size)
    return out


def rope(v, pos, theta) -> np.ndarray:
    """Rotates a copy of one head vector v[D] (or every row of v[..., D]) to position pos."""
    v = _f64(v).copy()
    d = v.shape[-1]
    flat = v.reshape(-1, d)
    for i in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[i])
        lib().or_rope(_ptr(row), d, int(pos), float(theta))
        flat[i] = row
    return flat.reshape(v.shape)


def _wtype(w, scale=None):
    """Weight type from the array and its scales: float32, uint16 (bf16 bits), int8 codes with
    per-row scales [n] (OR_I8) or per-group scales [n, k/128] (OR_I8G), or uint8 packed int4
    codes [n, k/2] with per-group scales (OR_I4G)."""
    if w.dtype == np.float32:
        return OR_F32
    if w.dtype == np.uint16:
        return OR_BF16
    if w.dtype == np.int8:
        return OR_I8G if scale is not None and np.ndim(scale) == 2 else OR_I8
    if w.dtype == np.uint8:
        return OR_I4G
    raise TypeError(f"unsupported weight dtype {w.dtype} (float32, uint16 bf16 bits, int8, uint8)")


def gemv(w, x, scale=None) -> np.ndarray:
    """y = W x; w is float32, uint16 (bf16 bits), int8 codes with scale [n] (per row) or
    [n, k/128] (per group), or uint8 packed int4 codes [n, k/2] with scale [n, k/128]."""
    w = np.ascontiguousarray(w)
    wt = _wtype(w, scale)
    n = w.shape[0]
    k = w.shape[1] * (2 if wt == OR_I4G else 1)
    x = _f64(x)
    assert x.size == k
    s = _f32(scale) if wt in (OR_I8, OR_I8G, OR_I4G) else None
    if wt in (OR_I8G, OR_I4G):
        assert k % GROUP == 0 and s.shape == (n, k // GROUP)
    y = np.empty(n, dtype=np.float64)
    lib().or_gemv(_ptr(w), wt, _ptr(s), _ptr(x), n, k, _ptr(y))
    return y


def quantize_rows(w):
    """Per-row symmetric int8: returns (codes int8 [n, k], scales float32 [n])."""
    w = _f32(w)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.int8)
    s = np.empty(n, dtype=np.float32)
    lib().or_quantize_rows(_ptr(w), n, k, _ptr(q), _ptr(s))
    return q, s


def quantize_groups(w, bits):
    """Group-wise symmetric quantisation with 128-value groups: bits = 8 returns (codes int8
    [n, k], scales float32 [n, k/128]); bits = 4 returns (packed uint8 [n, k/2], scales)."""
    assert bits in (8, 4)
    w = _f32(w)
    n, k = w.shape
    assert k % GROUP == 0
    q = np.empty((n, k) if bits == 8 else (n, k // 2), dtype=np.int8 if bits == 8 else np.uint8)
    s = np.empty((n, k // GROUP), dtype=np.float32)
    lib().or_quantize_groups(_ptr(w), n, k, bits, _ptr(q), _ptr(s))
    return q, s


def philox4x32_10(counter, key):
    """Philox4x32-10 block: counter (4 uint32), key (2 uint32) -> 4 uint32."""
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.empty(4, dtype=np.uint32)
    lib().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sample_uniform(seed, pos) -> float:
    """The uniform draw of the sampling step at position pos under seed (Philox4x32-10)."""
    return float(lib().or_sample_uniform(int(seed) & (2**64 - 1), int(pos)))


def sample(logits, temperature, top_p, u):
    """Temperature + top-p sampling by definition: (token, nucleus size, nucleus mass)."""
    z = _f64(logits)
    ns = C.c_int64(0)
    nm = C.c_double(0.0)
    tok = lib().or_sample(_ptr(z), z.size, float(temperature), float(top_p), float(u),
                          C.byref(ns), C.byref(nm))
    return int(tok), int(ns.value), float(nm.value)


def _attn_args(q, K, V):
    q = _f64(q)
    K = _f32(K)
    V = _f32(V)
    hq, d = q.shape
    t, hkv, d2 = K.shape
    assert d2 == d and V.shape == K.shape and hq % hkv == 0
    return q, K, V, t, hq, hkv, d


def attention(q, K, V) -> np.ndarray:
    """Two-pass causal GQA attention of q[Hq, D] over logical K, V [T, Hkv, D]."""
    q, K, V, t, hq, hkv, d = _attn_args(q, K, V)
    out = np.empty((hq, d), dtype=np.float64)
    lib().or_attention(_ptr(q), _ptr(K), _ptr(V), t, hq, hkv, d, _ptr(out))
    return out


def attention_online(q, K, V) -> np.ndarray:
    q, K, V, t, hq, hkv, d = _attn_args(q, K, V)
    out = np.empty((hq, d), dtype=np.float64)
    lib().or_attention_online(_ptr(q), _ptr(K), _ptr(V), t, hq, hkv, d, _ptr(out))
    return out


def attention_partitioned(q, K, V, part) -> np.ndarray:
    q, K, V, t, hq, hkv, d = _attn_args(q, K, V)
    out = np.empty((hq, d), dtype=np.float64)
    lib().or_attention_partitioned(_ptr(q), _ptr(K), _ptr(V), t, hq, hkv, d, int(part), _ptr(out))
    return out


def argmax(x) -> int:
    x = _f64(x)
    return int(lib().or_argmax(_ptr(x), x.size))


# ---- paged KV ---------------------------------------------------------------------------------

def pool_offset(pos, head, r, block_table, hkv, d, page) -> int:
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    return int(lib().or_pool_offset(pos, head, r, _ptr(bt), hkv, d, page))


def pool_scatter(logical, pos0, block_table, num_pages, page):
    """Expected pool contents (one layer, K or V) after writing logical [n, Hkv, D] rows at
    pos0..pos0+n-1; elements are copied bit for bit, untouched slots stay zero."""
    logical = np.ascontiguousarray(logical)
    n, hkv, d = logical.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    pool = np.zeros((num_pages, hkv, page, d), dtype=logical.dtype)
    lib().or_pool_scatter(_ptr(logical), logical.itemsize, pos0, n, _ptr(bt), hkv, d, page,
                          _ptr(pool))
    return pool


# ---- whole model --------------------------------------------------------------------------------

class _ORModel(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "qk_norm",
        "embed_type", "proj_type", "lm_type", "act_bf16", "kv_bf16", "logits_bf16",
        "max_ctx")] + [
        ("eps", C.c_double), ("theta", C.c_double),
        ("embed", C.c_void_p), ("lm_head", C.c_void_p), ("lm_scale", C.c_void_p),
        ("final_norm", C.c_void_p),
    ] + [(n, C.c_void_p) for n in (
        "qkv", "qkv_scale", "o", "o_scale", "gate_up", "gate_up_scale", "down", "down_scale",
        "in_norm", "post_norm", "q_norm", "k_norm", "k_cache", "v_cache")]


class Model:
    """Host-side model for ``or_decode_step``.

    ``weights`` is a dict: ``embed`` [V, d] (float32 or uint16 bf16 bits), ``lm_head`` (same
    convention, or quantised codes with ``lm_scale``; ``None`` when tied), ``final_norm`` [d]
    float32, and per-layer lists ``qkv``, ``o``, ``gate_up``, ``down`` (float32 / uint16 /
    quantised codes with ``*_scale`` lists, in the layouts ``gemv`` takes) and ``in_norm``,
    ``post_norm``, ``q_norm``, ``k_norm`` (float32).
    The KV cache is held here as logical float32 arrays [max_ctx, Hkv, D] per layer.
    """

    def __init__(self, cfg: dict, weights: dict, max_ctx: int):
        self.cfg = dict(cfg)
        self.w = weights
        L = cfg["n_layers"]
        hkv, d = cfg["n_kv_heads"], cfg["head_dim"]
        self.k_cache = [np.zeros((max_ctx, hkv, d), dtype=np.float32) for _ in range(L)]
        self.v_cache = [np.zeros((max_ctx, hkv, d), dtype=np.float32) for _ in range(L)]
        self._keep = []
        lm = weights.get("lm_head")
        if lm is None:
            lm = weights["embed"]
        s = _ORModel()
        s.n_layers, s.hidden = L, cfg["hidden"]
        s.n_q_heads, s.n_kv_heads, s.head_dim = cfg["n_q_heads"], hkv, d
        s.ffn, s.vocab, s.qk_norm = cfg["ffn"], cfg["vocab"], int(cfg.get("qk_norm", 1))
        s.embed_type = _wtype(weights["embed"])
        qs = weights.get("qkv_scale")
        s.proj_type = _wtype(weights["qkv"][0], qs[0] if qs else None)
        s.lm_type = _wtype(lm, weights.get("lm_scale"))
        s.act_bf16 = int(cfg["act_bf16"])
        s.kv_bf16 = int(cfg["kv_bf16"])
        s.logits_bf16 = int(cfg.get("logits_bf16", cfg["kv_bf16"]))
        s.max_ctx = max_ctx
        s.eps, s.theta = float(cfg["eps"]), float(cfg["theta"])
        s.embed = self._hold(weights["embed"])
        s.lm_head = self._hold(lm)
        s.lm_scale = (self._hold(_f32(weights.get("lm_scale")))
                      if s.lm_type in (OR_I8, OR_I8G, OR_I4G) else None)
        s.final_norm = self._hold(_f32(weights["final_norm"]))
        for key in ("qkv", "o", "gate_up", "down"):
            setattr(s, key, self._ptr_array([np.ascontiguousarray(a) for a in weights[key]]))
            sc = weights.get(key + "_scale")
            setattr(s, key + "_scale", self._ptr_array([_f32(a) for a in sc]) if sc else None)
        for key in ("in_norm", "post_norm", "q_norm", "k_norm"):
            setattr(s, key, self._ptr_array([_f32(a) for a in weights[key]]))
        s.k_cache = self._ptr_array(self.k_cache)
        s.v_cache = self._ptr_array(self.v_cache)
        self._s = s

    def _hold(self, a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        self._keep.append(a)
        return a.ctypes.data

    def _ptr_array(self, arrays):
        arr = (C.c_void_p * len(arrays))(*[self._hold(a) for a in arrays])
        self._keep.append(arr)
        return C.cast(arr, C.c_void_p).value

    def step(self, pos, token=None, embedding=None, want_logits=True):
        """Runs one decode step; returns (hidden [d] f64, logits [V] f64 or None, argmax or None)."""
        d, v = self.cfg["hidden"], self.cfg["vocab"]
        hidden = np.empty(d, dtype=np.float64)
        logits = np.empty(v, dtype=np.float64) if want_logits else None
        am = C.c_int32(-1)
        emb = _f64(embedding) if embedding is not None else None
        rc = lib().or_decode_step(C.byref(self._s), -1 if token is None else int(token), _ptr(emb),
                                  int(pos), _ptr(hidden), _ptr(logits),
                                  C.byref(am) if want_logits else None)
        if rc != 0:
            raise ValueError("or_decode_step rejected its arguments")
        return hidden, logits, (am.value if want_logits else None)
