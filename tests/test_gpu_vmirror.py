"""prefill_attn_vmirror_ex: the chunks of one sequence in turn with a V mirror
kept by the caller, through the C ABI, against prefill_attn_ex and the oracle.

Each chunk passes the previous chunk's end as mirror_keys, so the call
rewrites only the new keys' tiles (and the tile of its last key).  Where
prefill_attn_ex also rewrites V into operand order (at least 8 query tiles)
both run the same kernels on the same operand bits and must agree bit for
bit; shorter chunks, which prefill_attn_ex runs on V in place, must agree
within the parity bars.  Every chunk is compared with the oracle on all of
its rows.  The chunk ends fall inside tiles (32 keys), and the cache rows
past the sequence hold NaN, so no chunk may read a key past its last one.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, device, to_device

pytestmark = pytest.mark.gpu

H, KVH, D = 8, 2, 512
# (T, start_pos) of the chunks of one sequence, in order
CHUNKS = [(640, 0), (700, 640), (1, 1340), (4, 1341), (300, 1345), (1203, 1645)]
CAP = 2900           # cache and mirror capacity (not a multiple of the tile)


def _sequence(dtype):
    L_end = CHUNKS[-1][0] + CHUNKS[-1][1]
    x = workloads.make_random(H, KVH, D, L_end, 0, capacity=CAP, std=0.5, seed=4242, dtype=dtype)
    k_store, v_store = x.k_store.copy(), x.v_store.copy()
    nan = np.array(np.nan, dtype=np.float32)
    if dtype != "f32":
        nan = np.frombuffer(np.array([0x7FC0], dtype=np.uint16).tobytes(), dtype=k_store.dtype)[0]
    k_store[:, L_end:] = nan
    v_store[:, L_end:] = nan
    return x, to_device(x.q_store, dtype), to_device(k_store, dtype), to_device(v_store, dtype)


def _call_ex(pa, q, k, v, T, sp):
    import torch
    ws_b = pa.workspace_bytes(q_dtype(q), T, sp, H, KVH, D, 0)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=device()) if ws_b else None
    out = torch.full((T, H * D), float("nan"), device=device())
    pa.prefill_attn_ex(q[sp:sp + T], H * D, k, v, CAP * D, out, H * D, T, sp, H, KVH, D, 0, workspace=ws)
    return out


def _call_mirror(pa, q, k, v, mirror, mirror_keys, T, sp):
    import torch
    ws_b = pa.workspace_bytes(q_dtype(q), T, sp, H, KVH, D, 0)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=device()) if ws_b else None
    out = torch.full((T, H * D), float("nan"), device=device())
    pa.prefill_attn_vmirror_ex(q[sp:sp + T], H * D, k, v, CAP * D, mirror, CAP, mirror_keys, out, H * D,
                               T, sp, H, KVH, D, workspace=ws)
    return out


def q_dtype(q):
    import torch
    return {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[q.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_vmirror_sequence(orc, dtype):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    pa.load()
    x, q, k, v = _sequence(dtype)
    nb = pa.vmirror_bytes(dtype, KVH, D, CAP)
    assert nb == KVH * ((CAP + 31) // 32) * 32 * D * 2
    mirror = torch.full((nb,), 0x7F, dtype=torch.uint8, device=device())   # garbage until written
    first = {}
    mk = 0
    for T, sp in CHUNKS:
        print(f"  vmirror {dtype} chunk T={T} start_pos={sp} mirror_keys={mk}", flush=True)
        a = _call_mirror(pa, q, k, v, mirror, mk, T, sp)
        b = _call_ex(pa, q, k, v, T, sp)
        torch.cuda.synchronize()
        a = a.cpu().numpy().reshape(T, H, D)
        b = b.cpu().numpy().reshape(T, H, D)
        nq = -(-T // (128 // (H // KVH)))
        if nq >= 8:
            assert a.tobytes() == b.tobytes(), f"T={T} sp={sp}: same kernels, different bits"
        else:
            assert_parity(a, b.astype(np.float64), dtype, f"vmirror vs ex {dtype} T{T} sp{sp}",
                          group="vmirror")
        ref = orc.attention(x.q_f32[sp:sp + T], x.k_f32, x.v_f32, T, sp, H, KVH, D, window=0,
                            kv_head_stride=CAP * D)
        assert_parity(a, ref, dtype, f"vmirror vs oracle {dtype} T{T} sp{sp}", group="vmirror")
        first[(T, sp)] = a
        mk = sp + T

    # an earlier chunk again, over a mirror that now holds keys past its end:
    # the tile of its last key is rewritten, the tiles past it are not read
    T, sp = CHUNKS[4]
    a = _call_mirror(pa, q, k, v, mirror, sp + T, T, sp)
    # a chunk with mirror_keys = 0 rewrites everything up to its end
    T2, sp2 = CHUNKS[1]
    c = _call_mirror(pa, q, k, v, mirror, 0, T2, sp2)
    torch.cuda.synchronize()
    assert a.cpu().numpy().reshape(T, H, D).tobytes() == first[(T, sp)].tobytes()
    assert c.cpu().numpy().reshape(T2, H, D).tobytes() == first[(T2, sp2)].tobytes()


def test_vmirror_not_needed_is_ex():
    """At a head_dim whose kernels read V in place the mirror plays no part:
    a null mirror is accepted and the result is prefill_attn_ex's, bit for bit."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    lib = pa.load()
    Hh, KV, Dd, T, sp = 32, 8, 128, 300, 500
    assert pa.vmirror_bytes("bf16", KV, Dd, 4096) == 0
    x = workloads.make_random(Hh, KV, Dd, T, sp, std=0.5, seed=77, dtype="bf16")
    q, k, v = (to_device(t, "bf16") for t in (x.q_store, x.k_store, x.v_store))
    L = sp + T
    ws_b = pa.workspace_bytes("bf16", T, sp, Hh, KV, Dd, 0)
    ws = torch.empty(max(ws_b, 256), dtype=torch.uint8, device=device())
    out_a = torch.full((T, Hh * Dd), float("nan"), device=device())
    out_b = torch.full((T, Hh * Dd), float("nan"), device=device())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.prefill_attn_vmirror_ex(pa.PA_DTYPE_BF16, q.data_ptr(), Hh * Dd, k.data_ptr(), v.data_ptr(),
                                     L * Dd, None, 0, 0, out_a.data_ptr(), Hh * Dd, pa.PA_DTYPE_F32, T, sp,
                                     Hh, KV, Dd, ws.data_ptr(), ws.numel(), stream)
    assert st == pa.PA_OK, pa.strerror(st)
    pa.prefill_attn_ex(q, Hh * Dd, k, v, L * Dd, out_b, Hh * Dd, T, sp, Hh, KV, Dd, 0,
                       workspace=ws if ws_b else None)
    torch.cuda.synchronize()
    assert out_a.cpu().numpy().tobytes() == out_b.cpu().numpy().tobytes()
