"""Parity of the HIP path with the fp64 oracle, through the C ABI.

Full comparisons at sizes the oracle finishes in seconds (many tiles and a
ragged tail), and every row of every chunk of the workloads at full size, in
the launch configuration the benchmark times (oracle outputs cached on disk
by oracle_cache).  Bars: max |gpu - oracle| <= 1e-4 for fp32 inputs, <= 2e-2
for bf16/fp16 (fp32 output), plus a relative-RMS bar (gpu_util.TOL_REL_RMS)."""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle_cache
import workloads
from gpu_util import assert_parity, device, run_packed, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import causal_gqa_attention_prefill_amd as pa
    assert torch.cuda.is_available(), "no GPU"
    pa.load()


# ---- full comparisons on small shapes ---------------------------------------

SMALL = []
for dtype, D in [("f32", 32), ("f32", 64), ("f32", 128), ("f32", 256),
                 ("bf16", 32), ("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512),
                 ("f16", 64), ("f16", 128), ("f16", 256), ("f16", 512)]:
    for (H, KVH), (T, sp), W in [((4, 2), (77, 0), 0), ((8, 2), (130, 300), 0), ((8, 8), (5, 37), 0),
                                 ((8, 1), (200, 41), 50), ((6, 3), (33, 100), 1), ((4, 4), (1, 0), 0)]:
        SMALL.append((dtype, D, H, KVH, T, sp, W))


@pytest.mark.parametrize("dtype,D,H,KVH,T,sp,W", SMALL,
                         ids=[f"{c[0]}-D{c[1]}-H{c[2]}/{c[3]}-T{c[4]}-sp{c[5]}-W{c[6]}" for c in SMALL])
def test_small_full(orc, dtype, D, H, KVH, T, sp, W):
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=T * 7 + sp + D + W, dtype=dtype)
    got = run_packed(x, T, sp, H, KVH, D, W)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W)
    assert_parity(got, ref, dtype, f"{dtype} D{D} {H}/{KVH} T{T} sp{sp} W{W}")


@pytest.mark.parametrize("dtype,D,H,KVH,T,sp,W", [("bf16", 64, 128, 1, 5, 40, 0), ("f16", 128, 96, 1, 3, 300, 0),
                                                  ("bf16", 256, 128, 1, 2, 100, 30), ("bf16", 512, 128, 2, 3, 77, 0),
                                                  ("f32", 32, 128, 1, 4, 9, 0)])
def test_largest_groups(orc, dtype, D, H, KVH, T, sp, W):
    """Query-head groups up to the work-group's 128 rows (one token per tile)."""
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=H + D + T, dtype=dtype)
    got = run_packed(x, T, sp, H, KVH, D, W)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W)
    assert_parity(got, ref, dtype, f"group {H // KVH} {dtype} D{D}")


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("bf16", 128), ("f16", 128), ("bf16", 256), ("f16", 256)])
def test_peaked_softmax(orc, dtype, D):
    """Q scaled up 16x: peaked rows, large running-max jumps and rescales (the
    reference max moves on later tiles too, shifting scores already computed)."""
    H, KVH, T, sp = 8, 2, 150, 420
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=11, dtype=dtype)
    q16 = x.q_f32 * np.float32(16.0)
    if dtype == "bf16":
        q_store = workloads.round_to_bf16_bits(q16)
        q16 = workloads.bf16_bits_to_f32(q_store)
    elif dtype == "f16":
        h = q16.astype(np.float16)
        q_store, q16 = h.view(np.uint16), h.astype(np.float32)
    else:
        q_store = q16
    got = run_packed(x, T, sp, H, KVH, D, 0, q_rows=q_store)
    ref = orc.attention(q16, x.k_f32, x.v_f32, T, sp, H, KVH, D)
    assert_parity(got, ref, dtype, f"{dtype} D{D} Qx16")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 128), ("bf16", 256)])
def test_late_running_max_jump(orc, dtype, D):
    """One key far into each row's range gets a score well above everything
    before it, so the reference max moves late in the key loop and every
    earlier contribution is rescaled; rows see it or not by the causal bound."""
    H, KVH, T, sp = 8, 2, 96, 700
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=23, dtype=dtype)
    qh = x.q_f32.reshape(T, H, D)
    k = x.k_f32.copy()
    j = sp + 40                                   # rows t >= 40 see this key
    for kh in range(KVH):
        k[kh, j] = 6.0 * np.sign(qh[50, kh * (H // KVH)])
    if dtype == "bf16":
        k_store = workloads.round_to_bf16_bits(k)
        k = workloads.bf16_bits_to_f32(k_store)
    else:
        h = k.astype(np.float16)
        k_store, k = h.view(np.uint16), h.astype(np.float32)
    x.k_store, x.k_f32 = k_store, k
    got = run_packed(x, T, sp, H, KVH, D, 0)
    ref = orc.attention(x.q_f32, k, x.v_f32, T, sp, H, KVH, D)
    assert_parity(got, ref, dtype, f"{dtype} D{D} late max jump")


def test_planted_keys_outside_band(orc):
    """Keys right past the causal bound and right before the window start get
    huge scores; none may leak into any row."""
    H, KVH, D, T, sp, W = 4, 2, 128, 64, 200, 40
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=5, dtype="f32")
    k = x.k_f32.copy()
    v = x.v_f32.copy()
    qh = x.q_f32.reshape(T, H, D)
    for t in (0, 17, 40):
        pos = sp + t
        for j in (pos + 1, pos - W):
            for kh in range(KVH):
                k[kh, j] = 20.0 * np.sign(qh[t, kh * (H // KVH)])
                v[kh, j] = 100.0
    x.k_store, x.v_store, x.k_f32, x.v_f32 = k, v, k, v
    got = run_packed(x, T, sp, H, KVH, D, W)
    ref = orc.attention(x.q_f32, k, v, T, sp, H, KVH, D, window=W)
    assert_parity(got, ref, "f32", "planted keys")


def test_closed_form_band_f32():
    """q = 0: every valid key equally likely; V[kh, j, :] = j + 1000*kh gives
    out = (lo + pos)/2 + 1000*kv_head(h) exactly up to fp32 rounding."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    for H, KVH, D, T, sp, W in ((8, 2, 64, 100, 0, 0), (8, 2, 64, 100, 900, 0), (8, 4, 128, 70, 500, 33),
                                (4, 1, 32, 40, 10, 1)):
        L = sp + T
        q = torch.zeros(T, H * D, device=device())
        k = torch.randn(KVH, L, D, device=device())
        v = (torch.arange(L, device=device(), dtype=torch.float32)[None, :, None]
             + 1000.0 * torch.arange(KVH, device=device(), dtype=torch.float32)[:, None, None]).expand(KVH, L, D).contiguous()
        out = torch.empty(T, H * D, device=device())
        pa.prefill_attn(q, k, v, out, T, sp, H, KVH, D, W)
        torch.cuda.synchronize()
        o = out.cpu().numpy().reshape(T, H, D)
        pos = sp + np.arange(T)
        lo = np.maximum(0, pos - W + 1) if W > 0 else np.zeros_like(pos)
        want = (lo + pos)[:, None, None] / 2.0 + 1000.0 * (np.arange(H) // (H // KVH))[None, :, None]
        err = np.abs(o - want).max()
        assert err <= 1e-6 * max(1.0, float(np.abs(want).max())), (H, KVH, D, T, sp, W, err)


# ---- strided form, capacity caches, non-finite tails, untouched padding --------

@pytest.mark.parametrize("dtype,D", [("f32", 128), ("bf16", 128), ("bf16", 512), ("f16", 256)])
def test_ex_strided_nan_tail(orc, dtype, D):
    """Q inside a fused QKV row (stride (H + 2 KVH) D), a cache allocated for
    more positions than L whose tail is NaN, and an output with padded rows:
    the NaN tail must never be read and the padding never written."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, T, sp, W = 8, 2, 90, 150, 0
    L, cap = sp + T, sp + T + 77
    x = workloads.make_random(H, KVH, D, T, sp, capacity=cap, std=0.5, seed=3, dtype=dtype)
    qs = (H + 2 * KVH) * D
    q_fused = np.zeros((T, qs), dtype=x.q_store.dtype)
    q_fused[:, :H * D] = x.q_store
    k_store, v_store = x.k_store.copy(), x.v_store.copy()
    nan_bits = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}[dtype]
    k_store[:, L:] = nan_bits
    v_store[:, L:] = nan_bits
    q = to_device(q_fused, dtype)
    k = to_device(k_store, dtype)
    v = to_device(v_store, dtype)
    ors = H * D + 16
    out = torch.full((T, ors), float("nan"), device=device())
    ws_bytes = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device()) if ws_bytes else None
    pa.prefill_attn_ex(q, qs, k, v, cap * D, out, ors, T, sp, H, KVH, D, W, workspace=ws)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isnan(o[:, H * D:]).all(), "padding written"
    got = o[:, :H * D].reshape(T, H, D)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W, kv_head_stride=cap * D)
    assert_parity(got, ref, dtype, f"ex {dtype} D{D}")


@pytest.mark.parametrize("dtype,D,layout,T", [("f32", 128, "linear", 100), ("bf16", 128, "linear", 100),
                                               ("bf16", 256, "linear", 100), ("f16", 512, "linear", 100),
                                               ("bf16", 512, "linear", 300), ("bf16", 256, "ring", 100),
                                               ("bf16", 128, "paged", 100)])
def test_window_nan_below_band(orc, dtype, D, layout, T):
    """A windowed chunk whose first KV tile starts below every row's band:
    the cache rows below the first query's window start (inside that tile)
    and past L hold NaN, and none of it may reach the output (those keys are
    valid for no row, so they must contribute exactly nothing).  T = 300 at
    head_dim 512 takes the operand-order V copy."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, sp, W = 8, 2, 1000, 300
    L = sp + T
    lo0 = sp - W + 1                                     # 701: inside the KV tile starting at 640
    cap = L + 40
    x = workloads.make_random(H, KVH, D, T, sp, capacity=cap, std=0.5, seed=29 + D, dtype=dtype)
    nan_bits = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}[dtype]
    k_store, v_store = x.k_store.copy(), x.v_store.copy()
    for a in (k_store, v_store):
        a[:, :lo0] = nan_bits
        a[:, L:] = nan_bits
    q = to_device(x.q_store, dtype)
    out = torch.full((T, H * D), float("nan"), device=device())
    ws_b = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=device()) if ws_b else None
    if layout == "linear":
        pa.prefill_attn_ex(q, H * D, to_device(k_store, dtype), to_device(v_store, dtype), cap * D, out,
                           H * D, T, sp, H, KVH, D, W, workspace=ws)
    elif layout == "ring":
        R = W + T - 1 + 5                                # slots beyond what the chunk reads hold NaN
        kr = workloads.ring_cache(k_store, R, L, nan_bits)
        vr = workloads.ring_cache(v_store, R, L, nan_bits)
        pa.prefill_attn_ring_ex(q, H * D, to_device(kr, dtype), to_device(vr, dtype), R * D, R, out,
                                H * D, T, sp, H, KVH, D, W, workspace=ws)
    else:
        ps = 64
        npages = -(-L // ps) + 3
        kp, table = workloads.paged_cache(k_store, ps, L, npages, 7, nan_bits)
        vp, _ = workloads.paged_cache(v_store, ps, L, npages, 7, nan_bits)
        pa.prefill_attn_paged_ex(q, H * D, to_device(kp, dtype), to_device(vp, dtype), ps,
                                 torch.from_numpy(table).to(device()), out, H * D, T, sp, H, KVH, D, W,
                                 workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(T, H, D)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W, kv_head_stride=cap * D)
    assert_parity(got, ref, dtype, f"nan-below-band {layout} {dtype} D{D}", group="nan_below_band")


def test_split_path(orc):
    """Few query tiles over a long cache: the plan splits the keys and merges."""
    import causal_gqa_attention_prefill_amd as pa
    for dtype, H, KVH, D, T, sp, W in (("bf16", 8, 8, 128, 64, 6000, 0), ("f32", 4, 4, 64, 40, 3000, 0),
                                       ("bf16", 8, 2, 256, 100, 5000, 700), ("f16", 4, 1, 512, 20, 4000, 0)):
        assert pa.plan(dtype, T, sp, H, KVH, D, W)["kv_splits"] > 1
        x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=sp, dtype=dtype)
        got = run_packed(x, T, sp, H, KVH, D, W)
        ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W)
        assert_parity(got, ref, dtype, f"split {dtype} D{D}")


def test_chunked_matches_one_shot(orc):
    """A prompt prefilled in chunks through a growing cache equals the rows of
    the one-shot prefill (both against the oracle), and T = 1 decode steps too."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, D, N = 8, 2, 128, 700
    x = workloads.make_random(H, KVH, D, N, 0, std=0.5, seed=21, dtype="bf16")
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, N, 0, H, KVH, D)
    k = to_device(x.k_store, "bf16")
    v = to_device(x.v_store, "bf16")
    start = 0
    for T in (256, 1, 200, 243):
        q = to_device(x.q_store[start:start + T], "bf16")
        out = torch.empty(T, H * D, device=device())
        ws_b = pa.workspace_bytes("bf16", T, start, H, KVH, D, 0)
        ws = torch.empty(ws_b, dtype=torch.uint8, device=device()) if ws_b else None
        pa.prefill_attn_ex(q, H * D, k, v, N * D, out, H * D, T, start, H, KVH, D, 0, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy().reshape(T, H, D), ref[start:start + T], "bf16", f"chunk at {start}")
        start += T


# one shape per kernel variant: (label, dtype, H, KVH, D, T, sp, W, layout, expected plan fields)
VARIANTS = [
    ("32-row", "bf16", 32, 8, 128, 4096, 100, 0, "linear", {"waves_per_workgroup": 4, "kv_splits": 1}),
    ("32-row split+merge", "bf16", 32, 8, 128, 300, 1000, 0, "linear", {"waves_per_workgroup": 4}),
    ("paired", "bf16", 32, 8, 128, 2048, 300, 0, "linear", {"waves_per_workgroup": 8, "keys_per_tile": 64}),
    ("16-row key halves", "bf16", 8, 4, 256, 2048, 5000, 1024, "linear",
     {"waves_per_workgroup": 8, "keys_per_tile": 32, "kv_splits": 1}),
    ("16-row V copy + merge", "bf16", 8, 2, 512, 512, 3000, 0, "linear", {"waves_per_workgroup": 8}),
    ("fp32", "f32", 32, 8, 128, 300, 200, 0, "linear", {"waves_per_workgroup": 4}),
    ("ring", "bf16", 8, 4, 256, 512, 3000, 700, "ring", {}),
    ("paged", "bf16", 8, 2, 512, 4, 3000, 0, "paged", {}),
    ("V mirror", "bf16", 8, 2, 512, 100, 3000, 0, "vmirror", {}),
]


@pytest.mark.parametrize("case", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_deterministic(orc, case):
    """Five runs of each kernel variant give the same bytes (and the oracle's
    result within the bars)."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    label, dtype, H, KVH, D, T, sp, W, layout, want = case
    plan = pa.plan(dtype, T, sp, H, KVH, D, W)
    for k, v in want.items():
        assert plan[k] == v, (label, plan)
    if label.endswith("merge"):
        assert plan["kv_splits"] > 1 and plan["workspace_bytes"] > 0, plan
    L = sp + T
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=T + sp + D, dtype=dtype)
    q = to_device(x.q_store, dtype)
    out = torch.empty(T, H * D, device=device())
    ws_b = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=device()) if ws_b else None
    if layout == "linear":
        call = pa.PreparedCall(q, H * D, to_device(x.k_store, dtype), to_device(x.v_store, dtype), L * D,
                               out, H * D, T, sp, H, KVH, D, W, workspace=ws)
    elif layout == "vmirror":
        k, v = to_device(x.k_store, dtype), to_device(x.v_store, dtype)
        mirror = torch.empty(pa.vmirror_bytes(dtype, KVH, D, L), dtype=torch.uint8, device=device())
        # the keys before the chunk, as earlier chunks would have left them
        pa.PreparedCall(q, H * D, k, v, L * D, out, H * D, T, sp, H, KVH, D, W, workspace=ws,
                        v_mirror=mirror, mirror_capacity=L, mirror_keys=0)()
        call = pa.PreparedCall(q, H * D, k, v, L * D, out, H * D, T, sp, H, KVH, D, W, workspace=ws,
                               v_mirror=mirror, mirror_capacity=L, mirror_keys=sp)
    elif layout == "ring":
        R = W + T - 1
        call = pa.PreparedCall(q, H * D, to_device(workloads.ring_cache(x.k_store, R, L, 0), dtype),
                               to_device(workloads.ring_cache(x.v_store, R, L, 0), dtype), R * D, out,
                               H * D, T, sp, H, KVH, D, W, workspace=ws, ring_slots=R)
    else:
        npages = -(-L // 256) + 2
        kp, table = workloads.paged_cache(x.k_store, 256, L, npages, 3, 0)
        vp, _ = workloads.paged_cache(x.v_store, 256, L, npages, 3, 0)
        call = pa.PreparedCall(q, H * D, to_device(kp, dtype), to_device(vp, dtype), 0, out, H * D, T,
                               sp, H, KVH, D, W, workspace=ws,
                               page_table=torch.from_numpy(table).to(device()), page_size=256)
    runs = []
    for _ in range(5):
        out.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        runs.append(out.cpu().numpy().copy())
    for r in runs[1:]:
        assert r.tobytes() == runs[0].tobytes(), f"{label}: runs differ"
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W)
    assert_parity(runs[0].reshape(T, H, D), ref, dtype, f"determinism {label}", group="determinism")


# ---- the five workloads at full size ----------------------------------------------

def _run_workload(orc, name):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl)
    H, KVH, D, W = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.window
    if not wl.ring and not wl.page_size:
        k = to_device(x.k_store, wl.dtype)
        v = to_device(x.v_store, wl.dtype)
    for ci, (T, sp) in enumerate(wl.chunks):
        q_store, q_f32 = x.q_rows(ci)
        q = to_device(q_store, wl.dtype)
        out = torch.empty(T, H * D, device=device())
        ws_b = pa.workspace_bytes(wl.dtype, T, sp, H, KVH, D, W)
        ws = torch.empty(ws_b, dtype=torch.uint8, device=device()) if ws_b else None
        if wl.page_size:
            L = sp + T
            npages = -(-L // wl.page_size) + 16
            nan = np.uint16(0x7FC0) if wl.dtype == "bf16" else np.uint16(0x7E00)
            kp, table = workloads.paged_cache(x.k_store, wl.page_size, L, npages, wl.seed, nan)
            vp, _ = workloads.paged_cache(x.v_store, wl.page_size, L, npages, wl.seed, nan)
            pa.prefill_attn_paged_ex(q, H * D, to_device(kp, wl.dtype), to_device(vp, wl.dtype),
                                     wl.page_size, torch.from_numpy(table).to(device()), out, H * D,
                                     T, sp, H, KVH, D, W, workspace=ws)
        elif wl.ring:
            # the ring as the cache writes up to this chunk's last key leave it
            nan = np.uint16(0x7FC0) if wl.dtype == "bf16" else np.uint16(0x7E00)
            k = to_device(workloads.ring_cache(x.k_store, wl.ring, sp + T, nan), wl.dtype)
            v = to_device(workloads.ring_cache(x.v_store, wl.ring, sp + T, nan), wl.dtype)
            pa.prefill_attn_ring_ex(q, H * D, k, v, wl.ring * D, wl.ring, out, H * D, T, sp, H, KVH,
                                    D, W, workspace=ws)
        else:
            pa.prefill_attn_ex(q, H * D, k, v, wl.capacity * D, out, H * D, T, sp, H, KVH, D, W,
                               workspace=ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(T, H, D)
        # every row of the chunk against the fp64 oracle (cached per workload,
        # seed and chunk)
        ref = oracle_cache.reference(name, ci, x)
        assert_parity(got, ref, wl.dtype, f"{name} chunk {ci} (all {T * H} rows)", group=name)


@pytest.mark.parametrize("dtype,T,sp", [("bf16", 2048, 300), ("f16", 2040, 64), ("bf16", 2017, 4000)])
def test_paired_query_tiles(orc, dtype, T, sp):
    """Causal grids that fill the GPU with their pairs fitting one per CU pair
    the long and the short query tile of a kv head in one work-group: an
    unaligned start, a ragged last tile (8 tokens, 1 token), fp16, against
    oracle rows from every pair."""
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, D = 32, 8, 128
    plan = pa.plan(dtype, T, sp, H, KVH, D)
    nq, tq = plan["query_tiles"], plan["tokens_per_tile"]
    assert plan["waves_per_workgroup"] == 8 and plan["kv_splits"] == 1
    assert plan["workgroups"] == (nq + 1) // 2 * KVH
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=T + sp, dtype=dtype)
    got = run_packed(x, T, sp, H, KVH, D, 0)
    # first and last token of every query tile, for three heads of each kv head
    ts = sorted({t for q in range(nq) for t in (q * tq, min(q * tq + tq, T) - 1)})
    heads = [h for kh in range(KVH) for h in (kh * 4, kh * 4 + 3)]
    rt = np.array([t for t in ts for h in heads[::3]] + [t for t in ts[::7] for h in heads])
    rh = np.array([h for t in ts for h in heads[::3]] + [h for t in ts[::7] for h in heads])
    ref = orc.rows(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, rt, rh)
    assert_parity(got[rt, rh], ref, dtype, f"paired {dtype} T{T} sp{sp} ({len(rt)} rows)")
    assert np.isfinite(got).all()


def test_workload_tiny_f32(orc):
    _run_workload(orc, "tiny_f32")


def test_workload_mistral_f32(orc):
    _run_workload(orc, "mistral_f32")


def test_workload_mistral_bf16_chunked(orc):
    _run_workload(orc, "mistral_bf16_chunked")


def test_workload_mistral_bf16_oneshot(orc):
    _run_workload(orc, "mistral_bf16_oneshot")


def test_workload_mistral_f16_chunked(orc):
    _run_workload(orc, "mistral_f16_chunked")


def test_workload_gemma_global_bf16(orc):
    _run_workload(orc, "gemma_global_bf16")


def test_workload_gemma_swa_bf16(orc):
    _run_workload(orc, "gemma_swa_bf16")


def test_workload_gemma_swa_bf16_ring(orc):
    _run_workload(orc, "gemma_swa_bf16_ring")


def test_workload_gemma_global_verify_paged(orc):
    _run_workload(orc, "gemma_global_verify_paged")
