"""Ring caches through the C ABI (prefill_attn_ring_ex) against the oracle.

A sliding-window layer keeps its K/V in a ring: the key of position pos is
written into slot pos % R (the TensorSharp page, section 4, requirement R4).
Here each chunk's keys are written into the ring on the host before the
call, older keys are overwritten, never-written slots hold NaN, and every
chunk's output is compared with the oracle over the plain linear cache (the
definition; the oracle's own ring form is pinned to it on the CPU)."""
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


def _call_ring(x, dtype, q_rows, kr, vr, R, T, sp, H, KVH, D, W):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    q = to_device(q_rows, dtype)
    k = to_device(kr, dtype)
    v = to_device(vr, dtype)
    out = torch.empty(T, H * D, device=device())
    nb = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
    pa.prefill_attn_ring_ex(q, H * D, k, v, R * D, R, out, H * D, T, sp, H, KVH, D, W, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(T, H, D)


CASES = [
    # dtype, D, H, KVH, window, chunk sizes, extra slots beyond window + max(T) - 1
    ("bf16", 256, 8, 4, 100, (64, 64, 33, 1, 130), 0),
    ("bf16", 128, 8, 2, 50, (40, 77, 1, 90), 5),
    ("f16", 512, 4, 1, 70, (50, 50, 50), 0),
    ("bf16", 32, 4, 2, 20, (30, 2, 45), 7),
    ("f32", 64, 4, 2, 33, (20, 45, 7), 2),
    ("f32", 256, 4, 4, 40, (41, 41), 0),
    # rings a whole number of KV tiles long (64 keys; 32 for the split-half kernel)
    ("bf16", 128, 8, 2, 65, (64, 64, 64, 64), 0),
    ("bf16", 256, 8, 4, 97, (64, 64, 64, 64), 0),
]


@pytest.mark.parametrize("dtype,D,H,KVH,W,chunks,extra", CASES,
                         ids=[f"{c[0]}-D{c[1]}-W{c[4]}-R+{c[6]}" for c in CASES])
def test_ring_chunk_loop(orc, dtype, D, H, KVH, W, chunks, extra):
    N = sum(chunks)
    R = W + max(chunks) - 1 + extra
    x = workloads.make_random(H, KVH, D, N, 0, std=0.5, seed=N + D + W, dtype=dtype)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, N, 0, H, KVH, D, window=W)
    kr = np.full((KVH, R, D), NAN_BITS[dtype], dtype=x.k_store.dtype)
    vr = np.full((KVH, R, D), NAN_BITS[dtype], dtype=x.v_store.dtype)
    start = 0
    for T in chunks:
        for j in range(start, start + T):          # the chunk's cache writes
            kr[:, j % R] = x.k_store[:, j]
            vr[:, j % R] = x.v_store[:, j]
        got = _call_ring(x, dtype, x.q_store[start:start + T], kr, vr, R, T, start, H, KVH, D, W)
        assert_parity(got, ref[start:start + T], dtype, f"ring {dtype} D{D} R{R} chunk at {start}")
        start += T


@pytest.mark.parametrize("dtype,D,W,N", [("bf16", 128, 40, 150), ("bf16", 256, 24, 100),
                                         ("f32", 64, 20, 90)])
def test_ring_decode_window_slots(orc, dtype, D, W, N):
    """T = 1 steps need only `window` slots: each step writes its key, then
    attends.  These rings are shorter than a KV tile, so one tile wraps
    around them more than once."""
    H, KVH = 8, 2
    x = workloads.make_random(H, KVH, D, N, 0, std=0.5, seed=77 + D, dtype=dtype)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, N, 0, H, KVH, D, window=W)
    kr = np.full((KVH, W, D), NAN_BITS[dtype], dtype=x.k_store.dtype)
    vr = kr.copy()
    for p in range(N):
        kr[:, p % W] = x.k_store[:, p]
        vr[:, p % W] = x.v_store[:, p]
        got = _call_ring(x, dtype, x.q_store[p:p + 1], kr, vr, W, 1, p, H, KVH, D, W)
        assert_parity(got, ref[p:p + 1], dtype, f"decode at {p}")


@pytest.mark.parametrize("dtype,D,R", [("bf16", 128, 1532), ("bf16", 256, 1532), ("f16", 512, 1532),
                                       ("f32", 128, 1532), ("bf16", 128, 1536), ("f16", 512, 1536)])
def test_ring_split_plan(orc, dtype, D, R):
    """Few query tiles over a long window: the plan splits the keys across
    work-groups (workspace, merge pass); the ring wraps inside a tile (1532
    slots) or between tiles (1536)."""
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, T, sp, W = 8, 8, 20, 5000, 1500
    L = sp + T
    assert pa.plan(dtype, T, sp, H, KVH, D, W)["kv_splits"] > 1
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=D + 5, dtype=dtype)
    kr = workloads.ring_cache(x.k_store, R, L, NAN_BITS[dtype])
    vr = workloads.ring_cache(x.v_store, R, L, NAN_BITS[dtype])
    got = _call_ring(x, dtype, x.q_store, kr, vr, R, T, sp, H, KVH, D, W)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W)
    assert_parity(got, ref, dtype, f"ring split {dtype} D{D}")


def test_ring_full_causal_paired(orc):
    """A ring that holds every key (window 0, ring_slots >= L) on a full causal
    grid: the plan pairs the long and the short query tile of each kv head in
    one work-group (the ring form of the eight-wavefront kernel); slots past
    the last key hold NaN and are never read."""
    import causal_gqa_attention_prefill_amd as pa
    dtype, H, KVH, D, T, sp = "bf16", 32, 8, 128, 2048, 1000
    L = sp + T
    R = L + 77
    plan = pa.plan(dtype, T, sp, H, KVH, D)
    nq, tq = plan["query_tiles"], plan["tokens_per_tile"]
    assert plan["waves_per_workgroup"] == 8 and plan["workgroups"] == (nq + 1) // 2 * KVH
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=31, dtype=dtype)
    kr = workloads.ring_cache(x.k_store, R, L, NAN_BITS[dtype])
    vr = workloads.ring_cache(x.v_store, R, L, NAN_BITS[dtype])
    got = _call_ring(x, dtype, x.q_store, kr, vr, R, T, sp, H, KVH, D, 0)
    ts = sorted({t for qi in range(nq) for t in (qi * tq, min(qi * tq + tq, T) - 1)})
    heads = [kh * 4 + 2 for kh in range(KVH)]
    rt = np.array([t for t in ts for h in heads])
    rh = np.array([h for t in ts for h in heads])
    ref = orc.rows(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, rt, rh)
    assert_parity(got[rt, rh], ref, dtype, "ring paired")
    assert np.isfinite(got).all()
