"""The largest sizes the interface accepts.

* Positions up to 2^31 - 1 (the largest L, start_pos + T <= INT32_MAX) through
  a ring and a paged cache, whose memory is only the window's: the last KV
  tile then ends at 2^31, one past the largest int.
* Linear caches of the 16-bit kernels at their limit of one kv head's rows
  (0x7FE00000 bytes, the most the 32-bit buffer offsets address), and an fp32
  cache past 2 GiB per kv head (64-bit addressing).

The window keeps the oracle's work small: the output at positions
start_pos .. start_pos+T-1 depends only on the window's keys, so the oracle
runs on the last keys of the cache alone, shifted down to start at position
0 (the same bands, the same rows).  Those last keys also cover the KV tile
that holds the lowest window's first key (keys of a tile that fall outside
a row's band are masked, so they must hold the finite values a real cache
holds there); every row below that tile holds NaN, so a load of a tile
outside every band shows in the output.  Rings hold the keys their slots
hold after in-order writes."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, device, to_device

pytestmark = pytest.mark.gpu

INT32_MAX = 2 ** 31 - 1
MAX_HEAD_BYTES = 0x7FE00000
NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import causal_gqa_attention_prefill_amd as pa
    assert torch.cuda.is_available(), "no GPU"
    pa.load()


def _window_inputs(dtype, D, H, KVH, T, W, older, seed):
    """The T queries and the last older + W + T - 1 keys of the cache (the
    windows' keys and `older` keys below them), generated in the oracle's
    frame: keys at positions 0 .., queries at positions older + W - 1 .."""
    return workloads.make_random(H, KVH, D, T, older + W - 1, std=0.5, seed=seed, dtype=dtype)


def _oracle(orc, x, T, W, older, H, KVH, D):
    return orc.attention(x.q_f32, x.k_f32, x.v_f32, T, older + W - 1, H, KVH, D, window=W)


def _older_than_window(L, n):
    """Keys below the lowest window's first key (L - n) down to one whole
    64-key tile below the tile that holds it."""
    return (L - n) - (((L - n) // 64) * 64 - 64)


def _torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def _nan_tensor(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=_torch_dtype(dtype), device=device())


RING_CASES = [
    # dtype, D, H, KVH, T, W, extra ring slots (0: exactly the window; else rounded up to 64)
    ("bf16", 128, 8, 2, 100, 300, 0),
    ("bf16", 128, 8, 2, 100, 300, 64),
    ("bf16", 256, 8, 4, 64, 200, 64),
    ("bf16", 512, 8, 2, 40, 100, 0),
    ("f32", 64, 4, 2, 50, 90, 0),
]


@pytest.mark.parametrize("dtype,D,H,KVH,T,W,extra", RING_CASES,
                         ids=[f"{c[0]}-D{c[1]}-T{c[4]}-W{c[5]}-R+{c[6]}" for c in RING_CASES])
def test_ring_at_the_largest_positions(orc, dtype, D, H, KVH, T, W, extra):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    L = INT32_MAX
    sp = L - T
    n = W + T - 1
    R = n if extra == 0 else -(-n // 64) * 64 + extra
    # after in-order writes slot j % R holds key j for the last R keys
    x = _window_inputs(dtype, D, H, KVH, T, W, R - n, seed=D + T + extra)
    slots = (L - R + np.arange(R, dtype=np.int64)) % R
    kr = np.empty((KVH, R, D), dtype=x.k_store.dtype)
    vr = np.empty((KVH, R, D), dtype=x.v_store.dtype)
    kr[:, slots] = x.k_store
    vr[:, slots] = x.v_store
    out = torch.empty(T, H * D, device=device())
    nb = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
    pa.prefill_attn_ring_ex(to_device(x.q_store, dtype), H * D, to_device(kr, dtype), to_device(vr, dtype),
                            R * D, R, out, H * D, T, sp, H, KVH, D, W, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy().reshape(T, H, D), _oracle(orc, x, T, W, R - n, H, KVH, D), dtype,
                  f"ring of {R} slots ending at position {L - 1}")


PAGED_CASES = [
    # dtype, D, H, KVH, T, W, page size
    ("bf16", 128, 16, 4, 4, 500, 256),
    ("bf16", 128, 8, 2, 200, 400, 256),
    ("bf16", 512, 8, 2, 4, 300, 256),
    ("f32", 128, 8, 2, 3, 200, 256),
]


@pytest.mark.parametrize("dtype,D,H,KVH,T,W,P", PAGED_CASES,
                         ids=[f"{c[0]}-D{c[1]}-T{c[4]}-W{c[5]}-P{c[6]}" for c in PAGED_CASES])
def test_paged_at_the_largest_positions(orc, dtype, D, H, KVH, T, W, P):
    """Pages of the window only: table entries of the blocks below it point off
    the pool (never read), the window's blocks sit in scrambled pool pages."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    L = INT32_MAX
    sp = L - T
    n = W + T - 1
    b_lo, b_hi = (L - n) // P, (L - 1) // P
    first = b_lo * P                       # the window's pages hold keys from here on
    x = _window_inputs(dtype, D, H, KVH, T, W, L - n - first, seed=D + T + P)
    nb_win = b_hi - b_lo + 1
    npages = nb_win + 3
    order = np.random.default_rng(T + W).permutation(npages)[:nb_win].astype(np.int32)
    table = np.full(b_hi + 1, npages + 100, dtype=np.int32)
    table[b_lo:] = order
    pools = []
    for src in (x.k_store, x.v_store):
        pool = np.full((npages, KVH, P, D), NAN_BITS[dtype], dtype=src.dtype)
        for i in range(L - first):
            j = first + i
            pool[table[j // P], :, j % P] = src[:, i]
        pools.append(pool)
    out = torch.empty(T, H * D, device=device())
    nbytes = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device()) if nbytes else None
    pa.prefill_attn_paged_ex(to_device(x.q_store, dtype), H * D, to_device(pools[0], dtype),
                             to_device(pools[1], dtype), P, torch.from_numpy(table).to(device()), out,
                             H * D, T, sp, H, KVH, D, W, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy().reshape(T, H, D), _oracle(orc, x, T, W, L - n - first, H, KVH, D),
                  dtype, f"paged, {P}-position pages, ending at position {L - 1}")


LINEAR_CASES = [
    # dtype, D, H, KVH, T, W, cache rows per kv head
    ("bf16", 128, 4, 1, 300, 1000, MAX_HEAD_BYTES // (128 * 2)),
    ("bf16", 256, 2, 1, 256, 512, MAX_HEAD_BYTES // (256 * 2)),
    ("bf16", 512, 4, 1, 256, 300, MAX_HEAD_BYTES // (512 * 2)),     # with the V operand-order copy
    ("f16", 64, 4, 2, 100, 200, MAX_HEAD_BYTES // (64 * 2)),
    ("f32", 128, 4, 1, 200, 700, 5_000_000),                         # 2.56 GB per kv head
]


@pytest.mark.parametrize("dtype,D,H,KVH,T,W,L", LINEAR_CASES,
                         ids=[f"{c[0]}-D{c[1]}-T{c[4]}-W{c[5]}-L{c[6]}" for c in LINEAR_CASES])
def test_linear_at_the_size_limit(orc, dtype, D, H, KVH, T, W, L):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    sp = L - T
    n = W + T - 1
    older = _older_than_window(L, n)
    x = _window_inputs(dtype, D, H, KVH, T, W, older, seed=D + T + W)
    k = _nan_tensor((KVH, L, D), dtype)
    v = _nan_tensor((KVH, L, D), dtype)
    k[:, L - n - older:] = to_device(x.k_store, dtype)
    v[:, L - n - older:] = to_device(x.v_store, dtype)
    out = torch.empty(T, H * D, device=device())
    nb = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
    pa.prefill_attn_ex(to_device(x.q_store, dtype), H * D, k, v, L * D, out, H * D, T, sp, H, KVH, D, W,
                       workspace=ws)
    torch.cuda.synchronize()
    del k, v
    assert_parity(out.cpu().numpy().reshape(T, H, D), _oracle(orc, x, T, W, older, H, KVH, D), dtype,
                  f"linear cache of {L} rows per kv head")
    torch.cuda.empty_cache()

