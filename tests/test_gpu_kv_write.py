"""KV cache write (prefill_kv_write) through the C ABI: bit for bit against the
oracle's in-order writes, and chained with the attention the way a chunked
prefill runs it (write the chunk's K/V, then attend)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, device, to_device

pytestmark = pytest.mark.gpu

NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import causal_gqa_attention_prefill_amd as pa
    assert torch.cuda.is_available(), "no GPU"
    pa.load()


def _f32_image(store, dtype):
    if dtype == "f32":
        return np.asarray(store, dtype=np.float32)
    if dtype == "bf16":
        return workloads.bf16_bits_to_f32(store)
    return np.asarray(store, dtype=np.uint16).view(np.float16).astype(np.float32)


def _store(x, dtype):
    return workloads._to_storage(np.asarray(x, dtype=np.float32), dtype)[0]


def _from_device(t, dtype):
    import torch
    a = t.cpu()
    if dtype == "f32":
        return a.numpy()
    return a.view(torch.int16).numpy().view(np.uint16)


CASES = [
    # dtype, KVH, D, T, start_pos, ring slots (0: linear), extra source row elements
    ("bf16", 8, 128, 300, 1000, 0, 32 * 128),   # fused QKV rows: Q of 32 heads before K
    ("bf16", 4, 256, 200, 129000, 1024, 0),
    ("bf16", 4, 256, 2000, 5000, 777, 0),       # chunk longer than the ring
    ("f16", 2, 512, 65, 61440, 0, 0),
    ("f16", 2, 64, 50, 7, 16, 8),
    ("f32", 8, 128, 97, 3, 0, 0),
    ("f32", 2, 32, 40, 11, 9, 4),
]


@pytest.mark.parametrize("dtype,KVH,D,T,sp,R,extra", CASES,
                         ids=[f"{c[0]}-KVH{c[1]}-D{c[2]}-T{c[3]}-sp{c[4]}-R{c[5]}" for c in CASES])
def test_kv_write_bits(orc, dtype, KVH, D, T, sp, R, extra):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    rng = np.random.default_rng(T + D + R)
    srs = 2 * KVH * D + extra                 # [Q?][K][V] rows: K at extra, V after it
    rows_f = rng.standard_normal((T, srs), dtype=np.float32)
    rows = _store(rows_f, dtype)
    img = _f32_image(rows, dtype)
    rows_cache = R if R else sp + T + 5
    cache0 = np.full((KVH, rows_cache, D), NAN_BITS[dtype], dtype=rows.dtype)
    src = to_device(rows, dtype)
    kc = to_device(cache0, dtype)
    vc = to_device(cache0, dtype)
    flat = src.reshape(-1)                    # K and V sources: pointers into the rows
    pa.prefill_kv_write(flat[extra:], flat[extra + KVH * D:], srs, kc, vc, rows_cache * D, T, sp,
                        KVH, D, ring_slots=R)
    torch.cuda.synchronize()
    ko = np.full((KVH, rows_cache, D), np.nan, np.float32)
    vo = ko.copy()
    img_flat = np.ascontiguousarray(img).reshape(-1)
    orc.kv_write(img_flat[extra:], img_flat[extra + KVH * D:], srs, ko, vo, rows_cache * D, T, sp,
                 KVH, D, ring_slots=R)
    for got, want in ((kc, ko), (vc, vo)):
        g = _f32_image(_from_device(got, dtype), dtype)
        assert np.array_equal(g, want, equal_nan=True)


def test_kv_write_then_attend(orc):
    """A prompt prefilled chunk by chunk as the pages run it, entirely through the
    C ABI: each chunk's K/V rows (inside fused QKV rows) are written into a
    sliding-window ring and a global cache, then both layers attend; every
    chunk matches the oracle over the whole prompt."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, D, N, W = 8, 2, 128, 900, 256
    chunks = (300, 1, 256, 343)
    x = workloads.make_random(H, KVH, D, N, 0, std=0.5, seed=41, dtype="bf16")
    ref_g = orc.attention(x.q_f32, x.k_f32, x.v_f32, N, 0, H, KVH, D)
    ref_w = orc.attention(x.q_f32, x.k_f32, x.v_f32, N, 0, H, KVH, D, window=W)
    srs = (H + 2 * KVH) * D
    qkv = np.zeros((N, srs), np.uint16)
    qkv[:, :H * D] = x.q_store
    qkv[:, H * D:(H + KVH) * D] = x.k_store.transpose(1, 0, 2).reshape(N, KVH * D)
    qkv[:, (H + KVH) * D:] = x.v_store.transpose(1, 0, 2).reshape(N, KVH * D)
    qkv_d = to_device(qkv, "bf16")
    R = W + max(chunks) - 1
    nan = NAN_BITS["bf16"]
    kg = to_device(np.full((KVH, N, D), nan, np.uint16), "bf16")
    vg = to_device(np.full((KVH, N, D), nan, np.uint16), "bf16")
    kr = to_device(np.full((KVH, R, D), nan, np.uint16), "bf16")
    vr = to_device(np.full((KVH, R, D), nan, np.uint16), "bf16")
    start = 0
    for T in chunks:
        rows = qkv_d[start:start + T]
        k_src, v_src = rows.reshape(-1)[H * D:], rows.reshape(-1)[(H + KVH) * D:]
        pa.prefill_kv_write(k_src, v_src, srs, kg, vg, N * D, T, start, KVH, D)
        pa.prefill_kv_write(k_src, v_src, srs, kr, vr, R * D, T, start, KVH, D, ring_slots=R)
        outs = []
        for W_, kk, vv, stride, ring in ((0, kg, vg, N * D, None), (W, kr, vr, R * D, R)):
            out = torch.empty(T, H * D, device=device())
            nb = pa.workspace_bytes("bf16", T, start, H, KVH, D, W_)
            ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
            if ring is None:
                pa.prefill_attn_ex(rows, srs, kk, vv, stride, out, H * D, T, start, H, KVH, D, W_,
                                   workspace=ws)
            else:
                pa.prefill_attn_ring_ex(rows, srs, kk, vv, stride, ring, out, H * D, T, start, H,
                                        KVH, D, W_, workspace=ws)
            outs.append(out)
        torch.cuda.synchronize()
        assert_parity(outs[0].cpu().numpy().reshape(T, H, D), ref_g[start:start + T], "bf16",
                      f"global layer, chunk at {start}")
        assert_parity(outs[1].cpu().numpy().reshape(T, H, D), ref_w[start:start + T], "bf16",
                      f"window layer (ring {R}), chunk at {start}")
        start += T
