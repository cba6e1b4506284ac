"""Attention over host-resident K/V (qdec_offload_*) against the oracle and the resident path.

[ETE]'s KV-offload passage keeps the history K/V in host memory and copies one tile at a time into
device buffers, carrying the (m, l, acc) state across tiles.  The result is the attention of the
whole context, so the oracle is its plain two-pass definition.  Tiles are whole split-KV
partitions and their partials land in the resident path's slots, so with two or more partitions
the result must equal qdec_op_attention's bit for bit.  The host pages are laid out by the
oracle's pool addressing (identity page order), in pinned memory.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_step_04_amd import qdec as Q
from decode_step_04_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host_pages(logical):
    """Pinned host tensor of the page layout [pages][Hkv][16][D] (position order) of logical
    [T, Hkv, D] K or V (torch, bf16 or fp32)."""
    T = logical.shape[0]
    pages = (T + 15) // 16
    bt = np.arange(pages, dtype=np.int32)
    if logical.dtype == torch.bfloat16:
        arr = oracle.pool_scatter(synth.bf16_to_bits(logical), 0, bt, pages, 16)
        src = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        src = torch.from_numpy(oracle.pool_scatter(logical.cpu().numpy(), 0, bt, pages, 16))
    h = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
    h.copy_(src)
    return h


def _resident(q, kl, vl, hq, hkv, d, part):
    """qdec_op_attention on a device pool (identity block table) with partition `part`."""
    T = kl.shape[0]
    kp, vp = _host_pages(kl).to(DEV), _host_pages(vl).to(DEV)
    bt = torch.arange(kp.shape[0], dtype=torch.int32, device=DEV)
    wsb = Q.qdec_op_attention_workspace(T, hq, d, part)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    out = torch.empty((hq, d), device=DEV)
    kvt = Q.BF16 if kl.dtype == torch.bfloat16 else Q.F32
    Q.qdec_op_attention(q, Q.F32, kp, vp, kvt, bt, T, hq, hkv, d, part, ws, ws.numel(), out, Q.F32)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _offload(o, q, hk, hv, T, hq, d, out_dtype=Q.F32, stream=None):
    out = torch.empty((hq, d), device=DEV,
                      dtype=torch.float32 if out_dtype == Q.F32 else torch.bfloat16)
    Q.qdec_offload_attention(o, q, Q.BF16 if q.dtype == torch.bfloat16 else Q.F32, hk, hv, T, out,
                             out_dtype, stream)
    return out


CASES = [  # (D, Hq, Hkv, kv dtype, T, tile, slots, partition)
    (128, 16, 8, torch.bfloat16, 1, 512, 2, 0),
    (128, 16, 8, torch.bfloat16, 100, 64, 2, 64),
    (128, 16, 8, torch.bfloat16, 512, 512, 1, 128),
    (128, 16, 8, torch.bfloat16, 513, 512, 2, 128),
    (128, 32, 8, torch.bfloat16, 3000, 512, 3, 0),
    (128, 32, 8, torch.bfloat16, 3000, 256, 1, 64),
    (64, 4, 2, torch.float32, 777, 128, 2, 64),
    (64, 16, 2, torch.bfloat16, 2049, 1024, 2, 512),
    (128, 8, 8, torch.float32, 1000, 192, 4, 64),
    (128, 4, 1, torch.bfloat16, 5000, 2048, 8, 0),
    # n_slots 0: the kernel reads the mapped host pages directly
    (128, 16, 8, torch.bfloat16, 1, 512, 0, 0),
    (128, 32, 8, torch.bfloat16, 3000, 512, 0, 0),
    (64, 4, 2, torch.float32, 777, 128, 0, 64),
    (128, 8, 8, torch.float32, 1000, 192, 0, 64),
]


@pytest.mark.parametrize("d,hq,hkv,kvt,T,tile,slots,part", CASES)
def test_offload_matches_oracle_and_resident(d, hq, hkv, kvt, T, tile, slots, part):
    print(f"offload D={d} Hq={hq} Hkv={hkv} {kvt} T={T} tile={tile} slots={slots} part={part}",
          flush=True)
    g = torch.Generator(device=DEV).manual_seed(T + d + hq + tile)
    q = torch.randn((hq, d), generator=g, device=DEV) * 0.5
    kl = torch.randn((T, hkv, d), generator=g, device=DEV).to(kvt)
    vl = torch.randn((T, hkv, d), generator=g, device=DEV).to(kvt)
    o = Q.qdec_offload_create(hq, hkv, d, Q.BF16 if kvt == torch.bfloat16 else Q.F32, max(T, 4096),
                              tile, slots, part)
    try:
        _, p_eff = Q.qdec_offload_info(o)
        assert tile % p_eff == 0
        got = _offload(o, q, _host_pages(kl), _host_pages(vl), T, hq, d)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
    finally:
        Q.qdec_offload_destroy(o)
    ref = oracle.attention(q.cpu().numpy().astype(np.float64), kl.float().cpu().numpy(),
                           vl.float().cpu().numpy())
    assert np.max(np.abs(got - ref)) <= 1e-4
    if (T + p_eff - 1) // p_eff >= 2:
        res = _resident(q, kl, vl, hq, hkv, d, p_eff)
        assert np.array_equal(got, res)


def test_offload_full_size_128k():
    """The attention stress workload (32 Q / 8 KV heads, D 128, bf16 K/V, scores spanning about
    +-20) at 128K positions from host memory: 4096-position tiles in two buffers."""
    T = 131072
    print(f"offload stress T={T}", flush=True)
    q, kl, vl, _ = synth.attention_stress(T, device=DEV)
    hk, hv = _host_pages(kl), _host_pages(vl)
    ref = oracle.attention(q.cpu().numpy().astype(np.float64), kl.float().cpu().numpy(),
                           vl.float().cpu().numpy())
    res = _resident(q, kl, vl, 32, 8, 128, 512)
    for tile, slots in ((4096, 2), (512, 0)):
        o = Q.qdec_offload_create(32, 8, 128, Q.BF16, T, tile, slots, 512)
        try:
            got = _offload(o, q, hk, hv, T, 32, 128)
            torch.cuda.synchronize()
            got = got.cpu().numpy()
        finally:
            Q.qdec_offload_destroy(o)
        assert np.max(np.abs(got - ref)) <= 1e-4
        assert np.array_equal(got, res)


def test_offload_back_to_back_calls_and_streams():
    """Calls on one object reuse its buffers and partials: issued back to back (different
    contexts, the second on another stream, no host synchronisation in between) each must still
    see only its own data."""
    hq, hkv, d = 16, 8, 128
    g = torch.Generator(device=DEV).manual_seed(9)
    o = Q.qdec_offload_create(hq, hkv, d, Q.BF16, 8192, 512, 2, 128)
    try:
        inputs = []
        for T in (5000, 700, 3333, 64):
            q = torch.randn((hq, d), generator=g, device=DEV)
            kl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
            vl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
            out = torch.empty((hq, d), device=DEV)
            inputs.append((T, q, kl, vl, out, _host_pages(kl), _host_pages(vl)))
        s2 = torch.cuda.Stream()
        torch.cuda.synchronize()
        for i, (T, q, _, _, out, hk, hv) in enumerate(inputs):
            st = s2 if i % 2 else torch.cuda.current_stream()
            Q.qdec_offload_attention(o, q, Q.F32, hk, hv, T, out, Q.F32, st.cuda_stream)
        torch.cuda.synchronize()
        for _, q, kl, vl, out, _, _ in inputs:
            ref = oracle.attention(q.cpu().numpy().astype(np.float64), kl.float().cpu().numpy(),
                                   vl.float().cpu().numpy())
            assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-4
    finally:
        Q.qdec_offload_destroy(o)


def test_offload_bf16_out():
    hq, hkv, d, T = 16, 8, 128, 1500
    g = torch.Generator(device=DEV).manual_seed(3)
    q = torch.randn((hq, d), generator=g, device=DEV).to(torch.bfloat16)
    kl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vl = torch.randn((T, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    o = Q.qdec_offload_create(hq, hkv, d, Q.BF16, T, 512, 2, 0)
    try:
        out = _offload(o, q, _host_pages(kl), _host_pages(vl), T, hq, d, out_dtype=Q.BF16)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
    finally:
        Q.qdec_offload_destroy(o)
    ref = oracle.attention(q.float().cpu().numpy().astype(np.float64), kl.float().cpu().numpy(),
                           vl.float().cpu().numpy())
    spacing = np.abs(ref) * 2.0**-8 + 1e-6
    assert np.all(np.abs(got - ref) <= spacing)


def test_offload_rejects():
    hq, hkv, d = 8, 8, 64
    for bad in (dict(tile_tokens=100), dict(tile_tokens=0), dict(n_slots=-1), dict(n_slots=9),
                dict(partition_size=192, tile_tokens=512), dict(head_dim=96), dict(max_context=0),
                dict(n_kv_heads=3), dict(kv_dtype=Q.I8_ROW)):
        kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, kv_dtype=Q.F32, max_context=1024,
                  tile_tokens=512, n_slots=2, partition_size=0)
        kw.update(bad)
        with pytest.raises(Q.QdecError):
            Q.qdec_offload_create(**kw)
    o = Q.qdec_offload_create(hq, hkv, d, Q.F32, 1024, 512, 2, 0)
    try:
        q = torch.zeros((hq, d), device=DEV)
        out = torch.empty((hq, d), device=DEV)
        pinned = torch.zeros((64, hkv, 16, d), pin_memory=True)
        pageable = torch.zeros((64, hkv, 16, d))
        device_kv = torch.zeros((64, hkv, 16, d), device=DEV)
        for hk, T in ((pageable, 100), (device_kv, 100), (pinned, 1025), (pinned, 0)):
            with pytest.raises(Q.QdecError):
                Q.qdec_offload_attention(o, q, Q.F32, hk, pinned, T, out, Q.F32)
        # a valid call still works after the rejected ones
        Q.qdec_offload_attention(o, q, Q.F32, pinned, pinned, 100, out, Q.F32)
        torch.cuda.synchronize()
        assert torch.all(out == 0)
    finally:
        Q.qdec_offload_destroy(o)
    p = Q.qdec_host_alloc(1 << 20)
    Q.qdec_host_free(p)
