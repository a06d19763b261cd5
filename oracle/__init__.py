"""Oracle for chunked causal grouped-query prefill attention (fp64, CPU).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library and its Python
binding never import it, and it imports nothing from them.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one row at a time); this
module builds it with gcc and marshals numpy arrays.  The definition it
follows is the gnosis handoff page "Prefill attention -> GPU: handoff",
section "GPU design (the real fix)", with the sliding-window band of the
TensorSharp page "Design: closing the Gemma-4 long-prompt prefill gap",
section 5 (Option A); ``oracle.c`` spells out each step and its source.

Parity pins: every entry point here is pinned by the ``not gpu`` tests in
``tests/test_oracle_pins.py`` (brute force, a library routine, closed forms
and invariants) and by planted mistakes in ``tests/test_oracle_mutants.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile ``source`` into the shared library ``output`` with gcc."""
    tmp = output + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def default_threads() -> int:
    """Worker threads: OMP_NUM_THREADS when set, else every visible core."""
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


_I64 = ctypes.c_int64
_INT = ctypes.c_int
_FP = ctypes.POINTER(ctypes.c_float)
_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int32)


def _f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"oracle inputs are fp32 images, got {a.dtype}")
    return a


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


class Oracle:
    """ctypes front end of one build of ``oracle.c`` (tests load planted copies too)."""

    def __init__(self, library: str = LIBRARY):
        if library == LIBRARY and not os.path.exists(LIBRARY):
            build()
        self.path = library
        lib = ctypes.CDLL(library)
        lib.oracle_prefill_attention.argtypes = [
            _FP, _I64, _FP, _FP, _I64, _DP, _INT, _INT, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_prefill_attention.restype = _INT
        lib.oracle_prefill_attention_rows.argtypes = [
            _FP, _I64, _FP, _FP, _I64, _IP, _IP, _I64, _DP,
            _INT, _INT, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_prefill_attention_rows.restype = _INT
        lib.oracle_row_probabilities.argtypes = [
            _FP, _I64, _FP, _FP, _I64, _INT, _INT, _DP, ctypes.POINTER(_INT),
            _INT, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_row_probabilities.restype = _INT
        lib.oracle_prefill_attention_ring.argtypes = [
            _FP, _I64, _FP, _FP, _I64, _INT, _DP, _INT, _INT, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_prefill_attention_ring.restype = _INT
        lib.oracle_prefill_attention_rows_ring.argtypes = [
            _FP, _I64, _FP, _FP, _I64, _INT, _IP, _IP, _I64, _DP,
            _INT, _INT, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_prefill_attention_rows_ring.restype = _INT
        lib.oracle_kv_write.argtypes = [_FP, _FP, _I64, _FP, _FP, _I64, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_prefill_attention_paged.argtypes = [
            _FP, _I64, _FP, _FP, _INT, _INT, _IP, _DP, _INT, _INT, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_prefill_attention_paged.restype = _INT
        lib.oracle_prefill_attention_rows_paged.argtypes = [
            _FP, _I64, _FP, _FP, _INT, _INT, _IP, _IP, _IP, _I64, _DP,
            _INT, _INT, _INT, _INT, _INT, _INT, _INT]
        lib.oracle_prefill_attention_rows_paged.restype = _INT
        lib.oracle_kv_write.restype = _INT
        self.lib = lib

    @staticmethod
    def _strides(q, k, T, start_pos, num_heads, head_dim, q_row_stride, kv_head_stride,
                 ring_slots=0):
        if q_row_stride is None:
            q_row_stride = num_heads * head_dim
        if kv_head_stride is None:
            kv_head_stride = (ring_slots or (start_pos + T)) * head_dim
        return int(q_row_stride), int(kv_head_stride)

    def attention(self, q, k, v, T, start_pos, num_heads, num_kv_heads, head_dim,
                  window=0, q_row_stride=None, kv_head_stride=None, nthreads=None, ring_slots=0):
        """Whole chunk; returns fp64 [T, num_heads, head_dim].  ring_slots > 0:
        k and v are ring caches, key j in slot j % ring_slots."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        qs, ks = self._strides(q, k, T, start_pos, num_heads, head_dim,
                               q_row_stride, kv_head_stride, ring_slots)
        _check_sizes(q, k, v, T, start_pos, num_heads, num_kv_heads, head_dim, qs, ks, ring_slots)
        out = np.empty((T, num_heads, head_dim), dtype=np.float64)
        if ring_slots:
            rc = self.lib.oracle_prefill_attention_ring(
                _ptr(q, _FP), qs, _ptr(k, _FP), _ptr(v, _FP), ks, int(ring_slots), _ptr(out, _DP),
                T, start_pos, num_heads, num_kv_heads, head_dim, window,
                nthreads or default_threads())
        else:
            rc = self.lib.oracle_prefill_attention(
                _ptr(q, _FP), qs, _ptr(k, _FP), _ptr(v, _FP), ks, _ptr(out, _DP),
                T, start_pos, num_heads, num_kv_heads, head_dim, window,
                nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_prefill_attention returned {rc}")
        return out

    def rows(self, q, k, v, T, start_pos, num_heads, num_kv_heads, head_dim, row_t, row_h,
             window=0, q_row_stride=None, kv_head_stride=None, nthreads=None, ring_slots=0):
        """Rows (row_t[i], row_h[i]) only; returns fp64 [len(row_t), head_dim]."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        qs, ks = self._strides(q, k, T, start_pos, num_heads, head_dim,
                               q_row_stride, kv_head_stride, ring_slots)
        _check_sizes(q, k, v, T, start_pos, num_heads, num_kv_heads, head_dim, qs, ks, ring_slots)
        rt = np.ascontiguousarray(row_t, dtype=np.int32)
        rh = np.ascontiguousarray(row_h, dtype=np.int32)
        if rt.shape != rh.shape or rt.ndim != 1:
            raise ValueError("row_t and row_h must be 1-D and of equal length")
        out = np.empty((rt.size, head_dim), dtype=np.float64)
        rc = self.lib.oracle_prefill_attention_rows_ring(
            _ptr(q, _FP), qs, _ptr(k, _FP), _ptr(v, _FP), ks, int(ring_slots), _ptr(rt, _IP),
            _ptr(rh, _IP), rt.size, _ptr(out, _DP), T, start_pos, num_heads, num_kv_heads,
            head_dim, window, nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_prefill_attention_rows returned {rc}")
        return out

    def row_probabilities(self, q, k, v, T, start_pos, num_heads, num_kv_heads, head_dim,
                          t, h, window=0, q_row_stride=None, kv_head_stride=None):
        """Softmax probabilities of row (t, h); returns (lo, fp64 array over keys lo..=pos)."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        qs, ks = self._strides(q, k, T, start_pos, num_heads, head_dim,
                               q_row_stride, kv_head_stride)
        _check_sizes(q, k, v, T, start_pos, num_heads, num_kv_heads, head_dim, qs, ks)
        probs = np.empty(start_pos + T, dtype=np.float64)
        first = _INT(0)
        n = self.lib.oracle_row_probabilities(
            _ptr(q, _FP), qs, _ptr(k, _FP), _ptr(v, _FP), ks, t, h, _ptr(probs, _DP),
            ctypes.byref(first), T, start_pos, num_heads, num_kv_heads, head_dim, window)
        if n < 0:
            raise ValueError(f"oracle_row_probabilities returned {n}")
        return first.value, probs[:n].copy()


    def _pool_args(self, k_pool, v_pool, page_table, page_size, T, start_pos, num_heads, num_kv_heads,
                   head_dim, q, qs):
        k_pool, v_pool = _f32(k_pool), _f32(v_pool)
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        page_elems = page_size * num_kv_heads * head_dim
        if k_pool.size % page_elems or v_pool.size != k_pool.size:
            raise ValueError("pools must hold whole pages of page_size x num_kv_heads x head_dim")
        if pt.size * page_size < start_pos + T:
            raise ValueError("the page table does not cover the keys")
        if q.size < (T - 1) * qs + num_heads * head_dim:
            raise ValueError("q too small")
        return k_pool, v_pool, pt, k_pool.size // page_elems

    def attention_paged(self, q, k_pool, v_pool, page_table, page_size, T, start_pos, num_heads,
                        num_kv_heads, head_dim, window=0, q_row_stride=None, nthreads=None):
        """Whole chunk over a paged cache (pools of pages of page_size positions of
        every kv head, key j in page page_table[j // page_size]); fp64 [T, H, D]."""
        q = _f32(q)
        qs = int(q_row_stride or num_heads * head_dim)
        k_pool, v_pool, pt, npages = self._pool_args(k_pool, v_pool, page_table, page_size, T,
                                                     start_pos, num_heads, num_kv_heads, head_dim, q, qs)
        out = np.empty((T, num_heads, head_dim), dtype=np.float64)
        rc = self.lib.oracle_prefill_attention_paged(
            _ptr(q, _FP), qs, _ptr(k_pool, _FP), _ptr(v_pool, _FP), page_size, npages, _ptr(pt, _IP),
            _ptr(out, _DP), T, start_pos, num_heads, num_kv_heads, head_dim, window,
            nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_prefill_attention_paged returned {rc}")
        return out

    def rows_paged(self, q, k_pool, v_pool, page_table, page_size, T, start_pos, num_heads,
                   num_kv_heads, head_dim, row_t, row_h, window=0, q_row_stride=None, nthreads=None):
        """Rows (row_t[i], row_h[i]) over a paged cache; fp64 [len(row_t), D]."""
        q = _f32(q)
        qs = int(q_row_stride or num_heads * head_dim)
        k_pool, v_pool, pt, npages = self._pool_args(k_pool, v_pool, page_table, page_size, T,
                                                     start_pos, num_heads, num_kv_heads, head_dim, q, qs)
        rt = np.ascontiguousarray(row_t, dtype=np.int32)
        rh = np.ascontiguousarray(row_h, dtype=np.int32)
        out = np.empty((rt.size, head_dim), dtype=np.float64)
        rc = self.lib.oracle_prefill_attention_rows_paged(
            _ptr(q, _FP), qs, _ptr(k_pool, _FP), _ptr(v_pool, _FP), page_size, npages, _ptr(pt, _IP),
            _ptr(rt, _IP), _ptr(rh, _IP), rt.size, _ptr(out, _DP), T, start_pos, num_heads,
            num_kv_heads, head_dim, window, nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_prefill_attention_rows_paged returned {rc}")
        return out

    def kv_write(self, k_src, v_src, src_row_stride, k_cache, v_cache, kv_head_stride, T,
                 start_pos, num_kv_heads, head_dim, ring_slots=0):
        """Store tokens 0..T-1 of k_src/v_src (fp32 images) in the caches, in
        order: row start_pos + i, or slot (start_pos + i) % ring_slots.  The
        caches (contiguous fp32 arrays) are updated in place."""
        k_src, v_src = _f32(k_src), _f32(v_src)
        for c in (k_cache, v_cache):
            if c.dtype != np.float32 or not c.flags["C_CONTIGUOUS"]:
                raise TypeError("caches must be contiguous float32 arrays")
        rows = ring_slots or (start_pos + T)
        need_src = (T - 1) * src_row_stride + num_kv_heads * head_dim
        need_c = (num_kv_heads - 1) * kv_head_stride + rows * head_dim
        if k_src.size < need_src or v_src.size < need_src:
            raise ValueError("sources too small")
        if k_cache.size < need_c or v_cache.size < need_c:
            raise ValueError("caches too small")
        rc = self.lib.oracle_kv_write(_ptr(k_src, _FP), _ptr(v_src, _FP), int(src_row_stride),
                                      _ptr(k_cache, _FP), _ptr(v_cache, _FP), int(kv_head_stride),
                                      int(ring_slots), T, start_pos, num_kv_heads, head_dim)
        if rc != 0:
            raise ValueError(f"oracle_kv_write returned {rc}")


def _check_sizes(q, k, v, T, start_pos, num_heads, num_kv_heads, head_dim, qs, ks, ring_slots=0):
    rows = ring_slots or (start_pos + T)
    need_q = (T - 1) * qs + num_heads * head_dim
    need_kv = (num_kv_heads - 1) * ks + rows * head_dim
    if q.size < need_q:
        raise ValueError(f"q holds {q.size} elements, the chunk needs {need_q}")
    if k.size < need_kv or v.size < need_kv:
        raise ValueError(f"k/v hold {k.size}/{v.size} elements, the cache needs {need_kv}")


_default = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` in this directory (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
