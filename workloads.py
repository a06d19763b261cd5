"""Seeded synthetic inputs for chunked causal GQA prefill attention.

Shared by the tests, the smoke check and the benchmark.  This module holds
no attention arithmetic: it draws Q, K and V, rounds them to the storage
type, and describes the workloads' shapes.  Both the oracle and the GPU path
consume exactly the values drawn here.

Recipe: ``numpy.random.default_rng(seed)``, ``standard_normal`` in float32,
drawn in the order Q, then K, then V, each multiplied by the workload's
standard deviation; bf16 / fp16 workloads round those fp32 values to the
storage type with round-to-nearest-even, and the oracle receives the rounded
values widened back to fp32 (exact).

Shapes follow the pages' workloads: the Mistral-7B prompt of the gnosis
handoff page (32 query heads / 8 kv heads, head_dim 128, a 1358-token prompt;
"Diagnosis" and "GPU design"), and the Gemma-4 prefill of the TensorSharp
design page (head_dim 512 global layers, 2048-token chunks, late chunks near
position 60k, KV padded to a multiple of 256, sliding-window layers;
sections 1, 2 and 5).  Head counts of the Gemma-shaped layers and the
1024-key window are not on the pages; they are fixed here.
"""
from __future__ import annotations

import dataclasses
from typing import Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                       # storage type of Q, K, V: "f32", "bf16" or "f16"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    window: int                      # 0: causal only
    chunks: Tuple[Tuple[int, int], ...]  # (T, start_pos) per call, in order
    capacity: int                    # cache rows per kv head
    std: float                       # inputs ~ N(0, 1) * std
    seed: int
    summary: str = ""
    ring: int = 0                    # > 0: the GPU reads K/V from a ring of this many slots
    page_size: int = 0               # > 0: the GPU reads K/V from a paged pool of this page size

    @property
    def q_tokens(self) -> int:
        """Query rows drawn: positions first_start .. last end."""
        return self.chunks[-1][1] + self.chunks[-1][0] - self.chunks[0][1]

    @property
    def first_pos(self) -> int:
        return self.chunks[0][1]

    @property
    def row_elems(self) -> int:
        return self.num_heads * self.head_dim


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", "f32", 4, 2, 32, 0, ((64, 0),), 64, 1.0, 101,
        "tiny fp32 causal GQA prefill, 4/2 heads, head_dim 32, T=64 at start_pos 0"),
    "mistral_f32": Workload(
        "mistral_f32", "f32", 32, 8, 128, 0, ((1358, 0),), 1358, 0.5, 102,
        "Mistral-7B-shaped fp32 prefill, 32/8 heads, head_dim 128, one T=1358 chunk"),
    "mistral_bf16_chunked": Workload(
        "mistral_bf16_chunked", "bf16", 32, 8, 128, 0,
        ((2048, 0), (2048, 2048), (2048, 4096), (2048, 6144)), 8192, 0.5, 103,
        "Mistral-7B-shaped bf16 prefill of an 8192-token prompt as four T=2048 chunks"),
    # the same prompt in one call (T = 8192 at start_pos 0): the one-shot side
    # of the chunked == one-shot invariant
    "mistral_bf16_oneshot": Workload(
        "mistral_bf16_oneshot", "bf16", 32, 8, 128, 0, ((8192, 0),), 8192, 0.5, 103,
        "Mistral-7B-shaped bf16 prefill of an 8192-token prompt in one T=8192 call"),
    # the same prompt, shapes and values with fp16 storage (the fp16 matrix path)
    "mistral_f16_chunked": Workload(
        "mistral_f16_chunked", "f16", 32, 8, 128, 0,
        ((2048, 0), (2048, 2048), (2048, 4096), (2048, 6144)), 8192, 0.5, 103,
        "Mistral-7B-shaped fp16 prefill of an 8192-token prompt as four T=2048 chunks"),
    "gemma_global_bf16": Workload(
        "gemma_global_bf16", "bf16", 8, 2, 512, 0, ((2048, 61440),), 63488, 0.3, 104,
        "Gemma-style global layer, 8/2 heads, head_dim 512, T=2048 at start_pos 61440"),
    "gemma_swa_bf16": Workload(
        "gemma_swa_bf16", "bf16", 8, 4, 256, 1024, ((2048, 129024),), 131072, 0.3, 105,
        "Gemma-style sliding-window layer, 8/4 heads, head_dim 256, window 1024, "
        "T=2048 at start_pos 129024"),
    # the same layer and values, its K/V held in a ring cache of 3072 slots
    # (window + T - 1 = 3071 keys are read at once)
    "gemma_swa_bf16_ring": Workload(
        "gemma_swa_bf16_ring", "bf16", 8, 4, 256, 1024, ((2048, 129024),), 131072, 0.3, 105,
        "Gemma-style sliding-window layer as gemma_swa_bf16, K/V in a ring cache of 3072 slots "
        "(key j in slot j % 3072)", ring=3072),
    # a verify step of three drafted tokens (T = 4) over the global layer's
    # 61440 cached keys, read through a page table of 256-position pages
    "gemma_global_verify_paged": Workload(
        "gemma_global_verify_paged", "bf16", 8, 2, 512, 0, ((4, 61440),), 61444, 0.3, 106,
        "Gemma-style global layer, 8/2 heads, head_dim 512: a T=4 verify step at start_pos 61440 "
        "over a paged cache of 256-position pages", page_size=256),
}


def ring_cache(rows: np.ndarray, ring_slots: int, L: int, fill) -> np.ndarray:
    """The ring cache left by writing keys 0 .. L-1 of ``rows`` ([kv heads,
    positions, head_dim]) one after another into slot pos % ring_slots: slot s
    holds the newest key j < L with j % ring_slots == s; slots no key reached
    hold ``fill``."""
    kvh, _, d = rows.shape
    ring = np.full((kvh, ring_slots, d), fill, dtype=rows.dtype)
    first = max(0, L - ring_slots)
    j = np.arange(first, L)
    ring[:, j % ring_slots] = rows[:, first:L]
    return ring


def paged_cache(rows: np.ndarray, page_size: int, L: int, num_pages: int, seed: int, fill):
    """A paged cache holding keys 0 .. L-1 of ``rows`` ([kv heads, positions,
    head_dim]): a pool of ``num_pages`` pages ([num_pages, kv heads, page_size,
    head_dim]), the sequence's pages drawn in a seeded random order from the
    pool, and its page table (int32, one entry per page_size keys).  Pool rows
    that hold no key of the sequence hold ``fill``."""
    kvh, _, d = rows.shape
    n = (L + page_size - 1) // page_size
    if n > num_pages:
        raise ValueError("pool too small")
    table = np.random.default_rng(seed).permutation(num_pages)[:n].astype(np.int32)
    pool = np.full((num_pages, kvh, page_size, d), fill, dtype=rows.dtype)
    for b in range(n):
        j0, j1 = b * page_size, min(L, (b + 1) * page_size)
        pool[table[b], :, :j1 - j0] = rows[:, j0:j1]
    return pool, table


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Inputs:
    """Q, K, V of one workload.

    ``q``  [q_tokens, num_heads*head_dim]   (row stride = num_heads*head_dim)
    ``k``, ``v`` [num_kv_heads, capacity, head_dim]
    ``*_f32`` are fp32 images of the stored values (for the oracle); ``*_store``
    are the arrays in the storage type (float32, or uint16 bit patterns of bf16
    or fp16) for the GPU.
    """

    def __init__(self, wl: Workload, q_store, k_store, v_store, q_f32, k_f32, v_f32):
        self.wl = wl
        self.q_store, self.k_store, self.v_store = q_store, k_store, v_store
        self.q_f32, self.k_f32, self.v_f32 = q_f32, k_f32, v_f32

    def q_rows(self, chunk_index: int):
        """(store, f32) views of the query rows of one chunk."""
        T, sp = self.wl.chunks[chunk_index]
        a = sp - self.wl.first_pos
        return self.q_store[a:a + T], self.q_f32[a:a + T]


def _to_storage(x: np.ndarray, dtype: str):
    if dtype == "f32":
        return x, x
    if dtype == "bf16":
        bits = round_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits)
    if dtype == "f16":
        h = x.astype(np.float16)
        return h.view(np.uint16), h.astype(np.float32)
    raise ValueError(dtype)


def make_inputs(wl: Workload, seed: int | None = None) -> Inputs:
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    q = rng.standard_normal((wl.q_tokens, wl.row_elems), dtype=np.float32) * np.float32(wl.std)
    k = rng.standard_normal((wl.num_kv_heads, wl.capacity, wl.head_dim), dtype=np.float32) * np.float32(wl.std)
    v = rng.standard_normal((wl.num_kv_heads, wl.capacity, wl.head_dim), dtype=np.float32) * np.float32(wl.std)
    qs, qf = _to_storage(q, wl.dtype)
    ks, kf = _to_storage(k, wl.dtype)
    vs, vf = _to_storage(v, wl.dtype)
    return Inputs(wl, qs, ks, vs, qf, kf, vf)


def make_random(num_heads, num_kv_heads, head_dim, T, start_pos, capacity=None, std=1.0,
                seed=0, dtype="f32", q_row_stride=None):
    """Free-form case for tests: returns an Inputs whose workload has one chunk."""
    capacity = capacity or (start_pos + T)
    wl = Workload(f"random_{seed}", dtype, num_heads, num_kv_heads, head_dim, 0,
                  ((T, start_pos),), capacity, std, seed)
    rng = np.random.default_rng(seed)
    qrs = q_row_stride or num_heads * head_dim
    q = rng.standard_normal((T, qrs), dtype=np.float32) * np.float32(std)
    k = rng.standard_normal((num_kv_heads, capacity, head_dim), dtype=np.float32) * np.float32(std)
    v = rng.standard_normal((num_kv_heads, capacity, head_dim), dtype=np.float32) * np.float32(std)
    qs, qf = _to_storage(q, dtype)
    ks, kf = _to_storage(k, dtype)
    vs, vf = _to_storage(v, dtype)
    return Inputs(wl, qs, ks, vs, qf, kf, vf)

