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
