"""ctypes binding of libqdec.so (the C ABI declared in include/qdec.h).

Argument marshalling only: each function has the name of the C entry point it calls, converts
Python ints / tensors (anything with ``data_ptr()``) to pointers, and raises ``QdecError`` when
the call returns a status other than QDEC_OK.  Every computation happens in the library's HIP
kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqdec.so")
_lib = None

# qdec_status
OK, E_INVAL, E_UNSUPPORTED, E_STATE, E_RANGE, E_NOMEM, E_HIP = range(7)
# qdec_dtype
F32, BF16, I8_ROW, I8_G128, I4_G128 = 0, 1, 2, 3, 4
# qdec_weight
(W_EMBED, W_LM_HEAD, W_FINAL_NORM, W_IN_NORM, W_POST_NORM, W_Q_NORM, W_K_NORM, W_QKV, W_O,
 W_GATE_UP, W_DOWN) = range(11)
# qdec_kclass
K_NAMES = ("embed", "qkv", "rope_append", "attention", "merge", "o_proj", "gate_up", "down",
           "lm_head", "argmax")
K_COUNT = len(K_NAMES)


class QdecError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func}: status {status}: {message}")
        self.status = status


class qdec_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("tied_lm_head", C.c_int32), ("qk_norm", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("proj_dtype", C.c_int32),
                ("lm_head_dtype", C.c_int32), ("io_dtype", C.c_int32), ("act_dtype", C.c_int32),
                ("kv_dtype", C.c_int32),
                ("page_size", C.c_int32), ("num_pages", C.c_int32), ("max_context", C.c_int32),
                ("partition_size", C.c_int32), ("max_prefill", C.c_int32),
                ("weight_slots", C.c_int32)]


class qdec_step(C.Structure):
    _fields_ = [("token_embedding", C.c_void_p), ("token_id", C.c_void_p), ("pos", C.c_int32),
                ("reserved", C.c_int32), ("hidden_out", C.c_void_p), ("logits_out", C.c_void_p),
                ("argmax_out", C.c_void_p), ("temperature", C.c_float), ("top_p", C.c_float),
                ("seed", C.c_uint64)]


class qdec_info(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "params_per_layer", "params_total", "layer_matrix_bytes", "layer_scale_bytes",
        "lm_head_bytes", "kv_bytes_per_layer_token", "kv_pool_bytes", "device_bytes")] + [
        ("partition_tokens", C.c_int32), ("max_partitions", C.c_int32)]


class qdec_bytes(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "embed", "qkv", "rope_append", "attention", "merge", "o_proj", "gate_up", "down",
        "lm_head", "argmax", "total", "scratch")]


class qdec_offload_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "device", "n_q_heads", "n_kv_heads", "head_dim", "kv_dtype", "max_context", "tile_tokens",
        "n_slots", "partition_size")]


_P, _I32, _I64, _F, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
_SIGS = {
    "qdec_offload_create": [C.POINTER(qdec_offload_config), C.POINTER(_P)],
    "qdec_offload_destroy": [_P],
    "qdec_offload_info": [_P, C.POINTER(_I64), C.POINTER(_I32)],
    "qdec_offload_attention": [_P, _P, _I32, _P, _P, _I32, _P, _I32, _P],
    "qdec_offload_schedule": [_I32, _I32, C.POINTER(_I32), _I32, C.POINTER(_I32)],
    "qdec_host_alloc": [_SZ, C.POINTER(_P)],
    "qdec_host_free": [_P],
    "qdec_config_validate": [C.POINTER(qdec_config), C.c_char_p, _SZ],
    "qdec_config_info": [C.POINTER(qdec_config), C.POINTER(qdec_info)],
    "qdec_bytes_model": [C.POINTER(qdec_config), _I32, _I32, C.POINTER(qdec_bytes)],
    "qdec_create": [C.POINTER(qdec_config), _I32, C.POINTER(_P)],
    "qdec_destroy": [_P],
    "qdec_last_error": [_P],
    "qdec_status_string": [C.c_int],
    "qdec_info_get": [_P, C.POINTER(qdec_info)],
    "qdec_upload": [_P, _I32, _I32, _P, _I32, _I64, _I64, _I32, _P],
    "qdec_upload_i8": [_P, _I32, _I32, _P, _P, _I64, _I64, _I32, _P],
    "qdec_upload_quantized": [_P, _I32, _I32, _P, _P, _I64, _I64, _I32, _P],
    "qdec_weight_ptr": [_P, _I32, _I32, C.POINTER(_P), C.POINTER(_P)],
    "qdec_kv_set_block_table": [_P, _P, _I32, _P],
    "qdec_kv_write": [_P, _I32, _I32, _I32, _P, _P, _P],
    "qdec_kv_read": [_P, _I32, _I32, _I32, _P, _P, _P],
    "qdec_kv_pool_ptr": [_P, _I32, C.POINTER(_P), C.POINTER(_P)],
    "qdec_decode_step": [_P, C.POINTER(qdec_step), _P],
    "qdec_prefill": [_P, _P, _I32, _I32, _P, _P, _P, _P],
    "qdec_graph_capture": [_P, C.POINTER(qdec_step), _P],
    "qdec_graph_replay": [_P, _I32, _P],
    "qdec_graph_reset": [_P],
    "qdec_device_error": [_P, C.POINTER(_I32), _P],
    "qdec_profile_enable": [_P, _I32],
    "qdec_profile_collect": [_P, C.POINTER(C.c_double), C.POINTER(_I64)],
    "qdec_profile_kernel": [_P, _I32, _I32, _I32, C.POINTER(qdec_step), _P],
    "qdec_op_gemv": [_P, _I32, _P, _P, _I32, _P, _I32, _I64, _I64, _P],
    "qdec_op_quantize_rows": [_P, _I32, _P, _P, _I64, _I64, _P],
    "qdec_op_quantize_groups": [_P, _I32, _I32, _P, _P, _I64, _I64, _P],
    "qdec_op_gemm": [_P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _P],
    "qdec_op_prefill_attention": [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P],
    "qdec_op_sample": [_P, _I32, _I64, _F, _F, C.c_uint64, _I32, _P, _SZ, _P, _P],
    "qdec_op_sample_workspace": [_I64, C.POINTER(_SZ)],
    "qdec_op_rmsnorm": [_P, _P, _F, _P, _I32, _I32, _P],
    "qdec_op_rope_table": [_P, _I32, _I32, _F, _P],
    "qdec_op_qk_norm_rope_append": [_P, _P, _P, _F, _P, _I32, _P, _I32, _P, _P, _I32, _P, _I32,
                                    _I32, _I32, _I32, _P],
    "qdec_op_attention_workspace": [_I32, _I32, _I32, _I32, C.POINTER(_SZ)],
    "qdec_op_attention": [_P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _SZ,
                          _P, _I32, _P],
    "qdec_op_attention_noalloc": [_P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32,
                                  _I32, _P, _I32, _P],
    "qdec_op_argmax": [_P, _I32, _I64, _P, _P],
    "qdec_op_copy": [_P, _P, _I64, _P],
}
_VOID = {"qdec_destroy", "qdec_offload_destroy"}
_STR = {"qdec_last_error", "qdec_status_string"}


def lib():
    """The loaded library; raises if libqdec.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback path)")
        _lib = C.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(_lib, name)
            fn.argtypes = args
            fn.restype = None if name in _VOID else (C.c_char_p if name in _STR else C.c_int)
    return _lib


def exported_names():
    return list(_SIGS)


def _p(x):
    """Pointer value of an int, None, a ctypes object or a tensor (data_ptr())."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, C._SimpleCData):
        return x.value
    return C.cast(x, C.c_void_p).value


def _check(name, status, ctx=None):
    if status != OK:
        msg = lib().qdec_last_error(ctx).decode(errors="replace")
        raise QdecError(status, name, msg)


def _call(name, *args, ctx=None):
    _check(name, getattr(lib(), name)(*args), ctx)


# ---- configuration --------------------------------------------------------------------------

def make_config(**kw) -> qdec_config:
    c = qdec_config()
    c.page_size = 16
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def qdec_config_validate(cfg: qdec_config):
    buf = C.create_string_buffer(512)
    st = lib().qdec_config_validate(C.byref(cfg), buf, 512)
    return st, buf.value.decode()


def qdec_config_info(cfg: qdec_config) -> qdec_info:
    out = qdec_info()
    _call("qdec_config_info", C.byref(cfg), C.byref(out))
    return out


def qdec_bytes_model(cfg: qdec_config, context: int, with_logits: int = 1) -> qdec_bytes:
    out = qdec_bytes()
    _call("qdec_bytes_model", C.byref(cfg), context, with_logits, C.byref(out))
    return out


def qdec_status_string(status: int) -> str:
    return lib().qdec_status_string(status).decode()


# ---- lifecycle ----------------------------------------------------------------------------------

def qdec_create(cfg: qdec_config, device: int = 0) -> int:
    h = C.c_void_p()
    _call("qdec_create", C.byref(cfg), device, C.byref(h))
    return h.value


def qdec_destroy(ctx: int) -> None:
    lib().qdec_destroy(ctx)


def qdec_last_error(ctx=None) -> str:
    return lib().qdec_last_error(ctx).decode(errors="replace")


def qdec_info_get(ctx) -> qdec_info:
    out = qdec_info()
    _call("qdec_info_get", ctx, C.byref(out), ctx=ctx)
    return out


# ---- weights --------------------------------------------------------------------------------------

def qdec_upload(ctx, layer, which, src, src_dtype, rows, cols, src_is_device=1, stream=None):
    _call("qdec_upload", ctx, layer, which, _p(src), src_dtype, rows, cols, src_is_device,
          _p(stream), ctx=ctx)


def qdec_upload_i8(ctx, layer, which, codes, scales, rows, cols, src_is_device=1, stream=None):
    _call("qdec_upload_i8", ctx, layer, which, _p(codes), _p(scales), rows, cols, src_is_device,
          _p(stream), ctx=ctx)


def qdec_upload_quantized(ctx, layer, which, codes, scales, rows, cols, src_is_device=1,
                          stream=None):
    _call("qdec_upload_quantized", ctx, layer, which, _p(codes), _p(scales), rows, cols,
          src_is_device, _p(stream), ctx=ctx)


def qdec_weight_ptr(ctx, layer, which):
    d, s = C.c_void_p(), C.c_void_p()
    _call("qdec_weight_ptr", ctx, layer, which, C.byref(d), C.byref(s), ctx=ctx)
    return d.value, s.value


# ---- paged KV ---------------------------------------------------------------------------------------

def qdec_kv_set_block_table(ctx, table, stream=None):
    import numpy as np

    t = np.ascontiguousarray(table, dtype=np.int32)
    _call("qdec_kv_set_block_table", ctx, t.ctypes.data, t.size, _p(stream), ctx=ctx)


def qdec_kv_write(ctx, layer, pos0, n, k, v, stream=None):
    _call("qdec_kv_write", ctx, layer, pos0, n, _p(k), _p(v), _p(stream), ctx=ctx)


def qdec_kv_read(ctx, layer, pos0, n, k, v, stream=None):
    _call("qdec_kv_read", ctx, layer, pos0, n, _p(k), _p(v), _p(stream), ctx=ctx)


def qdec_kv_pool_ptr(ctx, layer):
    k, v = C.c_void_p(), C.c_void_p()
    _call("qdec_kv_pool_ptr", ctx, layer, C.byref(k), C.byref(v), ctx=ctx)
    return k.value, v.value


# ---- the step -----------------------------------------------------------------------------------------

def make_step(pos, token_id=None, token_embedding=None, hidden_out=None, logits_out=None,
              argmax_out=None, temperature=0.0, top_p=1.0, seed=0) -> qdec_step:
    s = qdec_step()
    s.temperature = temperature
    s.top_p = top_p
    s.seed = int(seed) & (2**64 - 1)
    s.token_embedding = _p(token_embedding)
    s.token_id = _p(token_id)
    s.pos = pos
    s.reserved = 0
    s.hidden_out = _p(hidden_out)
    s.logits_out = _p(logits_out)
    s.argmax_out = _p(argmax_out)
    return s


def qdec_decode_step(ctx, step: qdec_step, stream=None):
    _call("qdec_decode_step", ctx, C.byref(step), _p(stream), ctx=ctx)


def qdec_prefill(ctx, token_ids, n_tokens, pos0, hidden_out=None, logits_out=None,
                 argmax_out=None, stream=None):
    _call("qdec_prefill", ctx, _p(token_ids), n_tokens, pos0, _p(hidden_out), _p(logits_out),
          _p(argmax_out), _p(stream), ctx=ctx)


def qdec_graph_capture(ctx, templ: qdec_step, stream=None):
    _call("qdec_graph_capture", ctx, C.byref(templ), _p(stream), ctx=ctx)


def qdec_graph_replay(ctx, pos, stream=None):
    _call("qdec_graph_replay", ctx, pos, _p(stream), ctx=ctx)


def qdec_graph_reset(ctx):
    _call("qdec_graph_reset", ctx, ctx=ctx)


def qdec_device_error(ctx, stream=None) -> int:
    f = C.c_int32()
    _call("qdec_device_error", ctx, C.byref(f), _p(stream), ctx=ctx)
    return f.value


def qdec_profile_enable(ctx, enable=1):
    _call("qdec_profile_enable", ctx, int(enable), ctx=ctx)


def qdec_profile_collect(ctx):
    ms = (C.c_double * K_COUNT)()
    n = (C.c_int64 * K_COUNT)()
    _call("qdec_profile_collect", ctx, ms, n, ctx=ctx)
    return {K_NAMES[i]: (ms[i], n[i]) for i in range(K_COUNT)}


def qdec_profile_kernel(ctx, kclass, layer, reps, step: qdec_step, stream=None):
    _call("qdec_profile_kernel", ctx, kclass, layer, reps, C.byref(step), _p(stream), ctx=ctx)


# ---- op-level entry points ------------------------------------------------------------------------------

def qdec_op_gemv(w, w_dtype, w_scale, x, x_dtype, y, y_dtype, n, k, stream=None):
    _call("qdec_op_gemv", _p(w), w_dtype, _p(w_scale), _p(x), x_dtype, _p(y), y_dtype, n, k,
          _p(stream))


def qdec_op_quantize_rows(w, w_dtype, codes, scales, n, k, stream=None):
    _call("qdec_op_quantize_rows", _p(w), w_dtype, _p(codes), _p(scales), n, k, _p(stream))


GEMM_STORE, GEMM_RESID, GEMM_SWIGLU = 0, 1, 2


def qdec_op_gemm(a, w, y, y_dtype, resid, epilogue, m, n, k, stream=None):
    _call("qdec_op_gemm", _p(a), _p(w), _p(y), y_dtype, _p(resid), epilogue, m, n, k, _p(stream))


def qdec_op_prefill_attention(q, k_pool, v_pool, block_table, pos0, n_tokens, n_q_heads,
                              n_kv_heads, head_dim, out, stream=None):
    _call("qdec_op_prefill_attention", _p(q), _p(k_pool), _p(v_pool), _p(block_table), pos0,
          n_tokens, n_q_heads, n_kv_heads, head_dim, _p(out), _p(stream))


def qdec_op_sample_workspace(n):
    b = C.c_size_t(0)
    _call("qdec_op_sample_workspace", n, C.byref(b))
    return b.value


def qdec_op_sample(logits, dtype, n, temperature, top_p, seed, position, workspace,
                   workspace_bytes, out, stream=None):
    _call("qdec_op_sample", _p(logits), dtype, n, temperature, top_p, int(seed) & (2**64 - 1),
          position, _p(workspace), workspace_bytes, _p(out), _p(stream))


def qdec_op_quantize_groups(w, w_dtype, dst_dtype, codes, scales, n, k, stream=None):
    _call("qdec_op_quantize_groups", _p(w), w_dtype, dst_dtype, _p(codes), _p(scales), n, k,
          _p(stream))


def qdec_op_rmsnorm(x, gamma, eps, y, y_dtype, n, stream=None):
    _call("qdec_op_rmsnorm", _p(x), _p(gamma), eps, _p(y), y_dtype, n, _p(stream))


def qdec_op_rope_table(table, max_pos, head_dim, theta, stream=None):
    _call("qdec_op_rope_table", _p(table), max_pos, head_dim, theta, _p(stream))


def qdec_op_qk_norm_rope_append(qkv, q_gamma, k_gamma, eps, table, pos, q_out, q_dtype, k_pool,
                                v_pool, kv_dtype, block_table, n_q_heads, n_kv_heads, head_dim,
                                page_size=16, stream=None):
    _call("qdec_op_qk_norm_rope_append", _p(qkv), _p(q_gamma), _p(k_gamma), eps, _p(table), pos,
          _p(q_out), q_dtype, _p(k_pool), _p(v_pool), kv_dtype, _p(block_table), n_q_heads,
          n_kv_heads, head_dim, page_size, _p(stream))


def qdec_op_attention_workspace(ctx_len, n_q_heads, head_dim, partition_size) -> int:
    b = C.c_size_t()
    _call("qdec_op_attention_workspace", ctx_len, n_q_heads, head_dim, partition_size, C.byref(b))
    return b.value


def qdec_op_attention(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, ctx_len, n_q_heads,
                      n_kv_heads, head_dim, partition_size, workspace, workspace_bytes, out,
                      out_dtype, page_size=16, stream=None):
    _call("qdec_op_attention", _p(q), q_dtype, _p(k_pool), _p(v_pool), kv_dtype, _p(block_table),
          ctx_len, n_q_heads, n_kv_heads, head_dim, page_size, partition_size, _p(workspace),
          workspace_bytes, _p(out), out_dtype, _p(stream))


def qdec_op_attention_noalloc(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, ctx_len,
                              n_q_heads, n_kv_heads, head_dim, partition_size, out, out_dtype,
                              page_size=16, stream=None):
    _call("qdec_op_attention_noalloc", _p(q), q_dtype, _p(k_pool), _p(v_pool), kv_dtype,
          _p(block_table), ctx_len, n_q_heads, n_kv_heads, head_dim, page_size, partition_size,
          _p(out), out_dtype, _p(stream))


def qdec_op_argmax(x, x_dtype, n, out, stream=None):
    _call("qdec_op_argmax", _p(x), x_dtype, n, _p(out), _p(stream))


def qdec_op_copy(dst, src, nbytes, stream=None):
    _call("qdec_op_copy", _p(dst), _p(src), nbytes, _p(stream))


# ---- attention over host-resident K/V ----

def qdec_offload_create(n_q_heads, n_kv_heads, head_dim, kv_dtype, max_context, tile_tokens,
                        n_slots=2, partition_size=0, device=0) -> int:
    cfg = qdec_offload_config(device, n_q_heads, n_kv_heads, head_dim, kv_dtype, max_context,
                              tile_tokens, n_slots, partition_size)
    h = C.c_void_p()
    _call("qdec_offload_create", C.byref(cfg), C.byref(h))
    return h.value


def qdec_offload_destroy(o) -> None:
    lib().qdec_offload_destroy(o)


def qdec_offload_info(o):
    """(device bytes, partition length)."""
    b, p = C.c_int64(0), C.c_int32(0)
    _call("qdec_offload_info", o, C.byref(b), C.byref(p))
    return b.value, p.value


def qdec_offload_attention(o, q, q_dtype, host_k, host_v, ctx_len, out, out_dtype, stream=None):
    _call("qdec_offload_attention", o, _p(q), q_dtype, _p(host_k), _p(host_v), ctx_len, _p(out),
          out_dtype, _p(stream))


def qdec_offload_schedule(n_tiles, n_slots):
    """The enqueue order as a list of (kind, tile, slot, other) records."""
    n = C.c_int32(0)
    _call("qdec_offload_schedule", n_tiles, n_slots, None, 0, C.byref(n))
    buf = (C.c_int32 * (4 * n.value))()
    _call("qdec_offload_schedule", n_tiles, n_slots, buf, n.value, C.byref(n))
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n.value)]


def qdec_host_alloc(nbytes) -> int:
    p = C.c_void_p()
    _call("qdec_host_alloc", nbytes, C.byref(p))
    return p.value


def qdec_host_free(p) -> None:
    _call("qdec_host_free", p)
