"""Paged caches through the C ABI (prefill_attn_paged_ex) against the oracle.

Short chunks and decode steps over long contexts, as a draft or verify step
reads the target's [0, cached_len) keys through the sequence's page table
(the FreeToken page "perf(spec): capture the gemma4 assistant draft in cuda
graphs"), plus prefill chunks through pages.  Pages sit in scrambled pool
order, unused pool rows hold NaN, and table entries of blocks no row reads
point off the pool; every output is compared with the oracle over the plain
linear cache (the definition; the oracle's own paged form is pinned to it)."""
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


CASES = [
    # dtype, D, H, KVH, T, start_pos, window, page size
    ("bf16", 128, 32, 8, 1, 8191, 0, 256),      # decode
    ("bf16", 128, 32, 8, 4, 8000, 0, 64),       # verify of three drafts
    ("bf16", 128, 32, 8, 16, 5000, 0, 128),
    ("bf16", 512, 8, 2, 4, 20000, 0, 256),      # head_dim 512: the V operand-order copy reads pages
    ("bf16", 256, 8, 4, 8, 10000, 1024, 64),    # window: blocks below it point off the pool
    ("f16", 64, 4, 1, 3, 3000, 0, 64),
    ("f32", 128, 8, 2, 2, 4000, 0, 128),
    ("bf16", 128, 8, 2, 300, 700, 0, 64),       # a prefill chunk through pages
    ("bf16", 256, 8, 4, 200, 900, 100, 128),
]


@pytest.mark.parametrize("dtype,D,H,KVH,T,sp,W,P", CASES,
                         ids=[f"{c[0]}-D{c[1]}-T{c[4]}-sp{c[5]}-W{c[6]}-P{c[7]}" for c in CASES])
def test_paged(orc, dtype, D, H, KVH, T, sp, W, P):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    L = sp + T
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=T + sp + D, dtype=dtype)
    n = -(-L // P)
    npages = n + 7
    kp, table = workloads.paged_cache(x.k_store, P, L, npages, seed=L, fill=NAN_BITS[dtype])
    vp, _ = workloads.paged_cache(x.v_store, P, L, npages, seed=L, fill=NAN_BITS[dtype])
    if W:
        lo_min = max(0, sp - W + 1)
        table[:lo_min // P] = npages + 100       # never read: off the pool
    q = to_device(x.q_store, dtype)
    out = torch.empty(T, H * D, device=device())
    nb = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
    pa.prefill_attn_paged_ex(q, H * D, to_device(kp, dtype), to_device(vp, dtype), P,
                             torch.from_numpy(table).to(device()), out, H * D, T, sp, H, KVH, D, W,
                             workspace=ws)
    torch.cuda.synchronize()
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W)
    assert_parity(out.cpu().numpy().reshape(T, H, D), ref, dtype, f"paged {dtype} D{D} T{T} P{P}")


def test_paged_table_rewritten_between_calls(orc):
    """The table is read by the kernels: moving the sequence's pages to other
    pool pages and rewriting the table (same device buffer, same prepared
    call) gives the same result."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    dtype, D, H, KVH, T, sp, P = "bf16", 128, 16, 4, 4, 3000, 64
    L = sp + T
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=5, dtype=dtype)
    ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D)
    npages = 2 * (-(-L // P))
    q = to_device(x.q_store, dtype)
    out = torch.empty(T, H * D, device=device())
    table_d = torch.empty(-(-L // P), dtype=torch.int32, device=device())
    kpool = torch.empty(npages * KVH * P * D, dtype=torch.bfloat16, device=device())
    vpool = torch.empty_like(kpool)
    nb = pa.workspace_bytes(dtype, T, sp, H, KVH, D, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
    call = pa.PreparedCall(q, H * D, kpool, vpool, 0, out, H * D, T, sp, H, KVH, D, 0, workspace=ws,
                           page_table=table_d, page_size=P)
    for seed in (1, 2):
        kp, table = workloads.paged_cache(x.k_store, P, L, npages, seed=seed, fill=NAN_BITS[dtype])
        vp, _ = workloads.paged_cache(x.v_store, P, L, npages, seed=seed, fill=NAN_BITS[dtype])
        kpool.copy_(to_device(kp, dtype).reshape(-1))
        vpool.copy_(to_device(vp, dtype).reshape(-1))
        table_d.copy_(torch.from_numpy(table))
        call()
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy().reshape(T, H, D), ref, dtype, f"table {seed}")


@pytest.mark.parametrize("dtype,T,sp,P", [("bf16", 2048, 2048, 256), ("f16", 2030, 700, 64)])
def test_paged_prefill_paired(orc, dtype, T, sp, P):
    """A long causal prefill chunk through pages fills the GPU, so the plan
    pairs the long and the short query tile of each kv head in one
    work-group (the paged form of the eight-wavefront kernel); sampled rows
    of every pair against the oracle over the linear cache."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, D = 32, 8, 128
    plan = pa.plan(dtype, T, sp, H, KVH, D)
    nq, tq = plan["query_tiles"], plan["tokens_per_tile"]
    assert plan["waves_per_workgroup"] == 8 and plan["workgroups"] == (nq + 1) // 2 * KVH
    L = sp + T
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=T + sp, dtype=dtype)
    npages = -(-L // P) + 5
    kp, table = workloads.paged_cache(x.k_store, P, L, npages, seed=L, fill=NAN_BITS[dtype])
    vp, _ = workloads.paged_cache(x.v_store, P, L, npages, seed=L, fill=NAN_BITS[dtype])
    q = to_device(x.q_store, dtype)
    out = torch.empty(T, H * D, device=device())
    nb = pa.workspace_bytes(dtype, T, sp, H, KVH, D, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
    pa.prefill_attn_paged_ex(q, H * D, to_device(kp, dtype), to_device(vp, dtype), P,
                             torch.from_numpy(table).to(device()), out, H * D, T, sp, H, KVH, D, 0,
                             workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(T, H, D)
    ts = sorted({t for qi in range(nq) for t in (qi * tq, min(qi * tq + tq, T) - 1)})
    heads = [kh * 4 + 1 for kh in range(KVH)]
    rt = np.array([t for t in ts for h in heads])
    rh = np.array([h for t in ts for h in heads])
    ref = orc.rows(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, rt, rh)
    assert_parity(got[rt, rh], ref, dtype, f"paged paired {dtype} T{T} sp{sp} P{P}")
    assert np.isfinite(got).all()
