"""The packed entry points from several host threads, each on its own stream.

Their scratch (the operand-order V copy and the split partials at head_dim
512) lives in a buffer per (device, stream) that grows on demand; growing it
must never free memory that work already enqueued still reads, and two
streams must never share one.  Two threads issue packed head_dim-512 calls
with growing chunk lengths (so each stream's buffer grows several times while
the other thread launches), and every result is held to the oracle."""
from __future__ import annotations

import threading

import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, device, to_device

pytestmark = pytest.mark.gpu


def test_two_threads_two_streams_growing(orc):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    pa.load()
    H, KVH, D, sp = 8, 2, 512, 1500
    lengths = [40, 300, 700, 1200]            # workspace grows with T at each step
    sizes = [pa.workspace_bytes("bf16", T, sp, H, KVH, D) for T in lengths]
    assert all(b > 0 for b in sizes) and sizes == sorted(sizes), sizes
    cases = {}
    for th in range(2):
        for T in lengths:
            x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=100 * th + T, dtype="bf16")
            cases[th, T] = (x, orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D))
    dev_in = {key: tuple(to_device(a, "bf16") for a in (x.q_store, x.k_store, x.v_store))
              for key, (x, _) in cases.items()}
    results, errors = {}, []

    def worker(th):
        try:
            s = torch.cuda.Stream()
            for rep in range(3):
                for T in lengths:
                    q, k, v = dev_in[th, T]
                    with torch.cuda.stream(s):
                        out = torch.empty(T, H * D, dtype=torch.float32, device=device())
                    pa.prefill_attn(q, k, v, out, T, sp, H, KVH, D, 0, stream=s)
                    s.synchronize()
                    results[th, T, rep] = out.cpu().numpy().reshape(T, H, D)
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(th,)) for th in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    for (th, T, rep), got in sorted(results.items()):
        _, ref = cases[th, T]
        assert_parity(got, ref, "bf16", f"threads t{th} T{T} rep{rep}", group="threads_streams")
    assert len(results) == 2 * 3 * len(lengths)
