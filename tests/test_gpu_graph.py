"""A fixed-shape chunk loop captured in one HIP graph through the C ABI.

The strided entry point with an explicit workspace allocates nothing,
synchronises nothing and clears no memory, so its launches can be recorded
into a graph (here through torch's capture of a side stream).  Each replay
must give the bits the eager calls give; replays alternate with eager work
and synchronisations, and the outputs are cleared between replays."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, device, to_device

pytestmark = pytest.mark.gpu


def test_graph_replay_of_chunk_loop(orc):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    pa.load()
    H, KVH, D, N = 8, 2, 128, 1100
    x = workloads.make_random(H, KVH, D, N, 0, std=0.5, seed=31, dtype="bf16")
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, N, 0, H, KVH, D)
    k = to_device(x.k_store, "bf16")
    v = to_device(x.v_store, "bf16")
    side = torch.cuda.Stream()
    # three prefill chunks and a short tail whose plan splits the keys (workspace)
    chunks = [(256, 0), (300, 256), (520, 556), (24, 1076)]
    calls, outs = [], []
    for T, sp in chunks:
        q = to_device(x.q_store[sp:sp + T], "bf16")
        out = torch.empty(T, H * D, device=device())
        nb = pa.workspace_bytes("bf16", T, sp, H, KVH, D, 0)
        ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
        calls.append(pa.PreparedCall(q, H * D, k, v, N * D, out, H * D, T, sp, H, KVH, D, 0,
                                     workspace=ws, stream=side))
        outs.append(out)
    assert pa.plan("bf16", 24, 1076, H, KVH, D, 0)["kv_splits"] > 1

    def loop():
        for c in calls:
            c()

    with torch.cuda.stream(side):
        loop()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for (T, sp), o in zip(chunks, eager):
        assert_parity(o.cpu().numpy().reshape(T, H, D), ref[sp:sp + T], "bf16", f"eager chunk at {sp}")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        loop()
    torch.cuda.synchronize()
    for rep in range(4):
        with torch.cuda.stream(side):
            for o in outs:
                o.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {rep}, chunk {i}"
        with torch.cuda.stream(side):   # eager work between replays
            loop()
        torch.cuda.synchronize()


def test_graph_replay_over_lengths(orc):
    """One captured graph of a verify step (T = 4) over a paged cache, its start
    position in a device buffer that is rewritten before each replay together
    with the query rows and the cache contents (as the FreeToken page copies
    the cached length and pending tokens into fixed buffers): every replay, at
    lengths from 100 to 8000 keys, matches the oracle and the same call made
    with a host start_pos, bit for bit."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    pa.load()
    H, KVH, D, T, P = 16, 4, 128, 4, 256
    max_sp = 7996
    N = max_sp + T
    npages = -(-N // P) + 5
    x = workloads.make_random(H, KVH, D, N, 0, std=0.5, seed=51, dtype="bf16")
    nan = np.uint16(0x7FC0)
    _, table_full = workloads.paged_cache(x.k_store, P, N, npages, seed=9, fill=nan)
    side = torch.cuda.Stream()
    q_buf = torch.empty(T, H * D, dtype=torch.bfloat16, device=device())
    kpool = torch.empty(npages * KVH * P * D, dtype=torch.bfloat16, device=device())
    vpool = torch.empty_like(kpool)
    table = torch.from_numpy(table_full).to(device())
    sp_buf = torch.zeros(1, dtype=torch.int32, device=device())
    out = torch.empty(T, H * D, device=device())
    out_host = torch.empty_like(out)
    nb = pa.workspace_bytes("bf16", T, max_sp, H, KVH, D, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=device())
    dev_call = pa.PreparedCall(q_buf, H * D, kpool, vpool, 0, out, H * D, T, max_sp, H, KVH, D, 0,
                               workspace=ws, stream=side, page_table=table, page_size=P,
                               start_pos_dev=sp_buf)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dev_call()
    torch.cuda.synchronize()
    for sp in (100, 1234, 4000, max_sp):
        L = sp + T
        kp, _ = workloads.paged_cache(x.k_store[:, :L], P, L, npages, seed=9, fill=nan)
        vp, _ = workloads.paged_cache(x.v_store[:, :L], P, L, npages, seed=9, fill=nan)
        kpool.copy_(to_device(kp, "bf16").reshape(-1))
        vpool.copy_(to_device(vp, "bf16").reshape(-1))
        q_buf.copy_(to_device(x.q_store[sp:sp + T], "bf16"))
        sp_buf.fill_(sp)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            g.replay()
        torch.cuda.synchronize()
        ref = orc.attention(x.q_f32[sp:sp + T], x.k_f32[:, :L], x.v_f32[:, :L], T, sp, H, KVH, D,
                            kv_head_stride=L * D)
        got = out.cpu().numpy().reshape(T, H, D)
        assert_parity(got, ref, "bf16", f"replay at start_pos {sp}")
        nbh = pa.workspace_bytes("bf16", T, sp, H, KVH, D, 0)
        wsh = torch.empty(nbh, dtype=torch.uint8, device=device()) if nbh else None
        pa.prefill_attn_paged_ex(q_buf, H * D, kpool, vpool, P, table, out_host, H * D, T, sp, H,
                                 KVH, D, 0, workspace=wsh)
        torch.cuda.synchronize()
        if pa.plan("bf16", T, sp, H, KVH, D, 0)["kv_splits"] == pa.plan("bf16", T, max_sp, H, KVH, D, 0)["kv_splits"]:
            assert torch.equal(out, out_host), sp
        else:
            assert_parity(out_host.cpu().numpy().reshape(T, H, D), ref, "bf16", f"host start {sp}")


def test_graph_replay_of_vmirror_loop(orc):
    """The same kind of loop at head_dim 512 through the V mirror (each chunk
    passes its start as mirror_keys, so the graph also rewrites the mirror's
    new tiles): replays give the eager bits, and the eager results match the
    oracle."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    pa.load()
    H, KVH, D, N = 8, 2, 512, 1100
    x = workloads.make_random(H, KVH, D, N, 0, std=0.5, seed=37, dtype="bf16")
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, N, 0, H, KVH, D)
    k = to_device(x.k_store, "bf16")
    v = to_device(x.v_store, "bf16")
    mirror = torch.empty(pa.vmirror_bytes("bf16", KVH, D, N), dtype=torch.uint8, device=device())
    side = torch.cuda.Stream()
    chunks = [(256, 0), (300, 256), (520, 556), (24, 1076)]
    calls, outs = [], []
    for T, sp in chunks:
        q = to_device(x.q_store[sp:sp + T], "bf16")
        out = torch.empty(T, H * D, device=device())
        nb = pa.workspace_bytes("bf16", T, sp, H, KVH, D, 0)
        ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
        calls.append(pa.PreparedCall(q, H * D, k, v, N * D, out, H * D, T, sp, H, KVH, D, 0,
                                     workspace=ws, stream=side, v_mirror=mirror, mirror_capacity=N,
                                     mirror_keys=sp))
        outs.append(out)

    def loop():
        for c in calls:
            c()

    with torch.cuda.stream(side):
        loop()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for (T, sp), o in zip(chunks, eager):
        assert_parity(o.cpu().numpy().reshape(T, H, D), ref[sp:sp + T], "bf16", f"vmirror eager chunk at {sp}",
                      group="graph")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        loop()
    torch.cuda.synchronize()
    for rep in range(4):
        with torch.cuda.stream(side):
            for o in outs:
                o.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {rep}, chunk {i}"
        with torch.cuda.stream(side):   # eager work between replays
            loop()
        torch.cuda.synchronize()
