"""Python binding of libprefill_attn.so (ctypes; argument marshalling only).

Every step of the attention runs in the HIP kernels of the library; this
module only turns torch tensors into pointers, strides and a stream, checks
that the tensors are large enough for the pointers it passes, and raises on
a non-zero status.  PyTorch supplies device memory and the current stream.
There is no fallback: when the library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libprefill_attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "prefill_attn.h")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_WORKSPACE = 0, 1, 2, 3, 4
PA_DTYPE_F32, PA_DTYPE_BF16, PA_DTYPE_F16 = 0, 1, 2
DTYPE_CODES = {"f32": PA_DTYPE_F32, "bf16": PA_DTYPE_BF16, "f16": PA_DTYPE_F16}
PLAN_FIELDS = ("tokens_per_tile", "query_tiles", "kv_splits", "workgroups", "keys_per_tile",
               "waves_per_workgroup", "workspace_bytes", "kv_tiles_visited")


class PrefillAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({strerror(status)})")


_lib = None


def library_path() -> str:
    return LIBRARY


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is missing: build it first (python -c "
                           "'import __graft_entry__; __graft_entry__.build()')")
    lib = ctypes.CDLL(LIBRARY)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    tail = [I, I, I, I, I, I, P]
    for name in ("prefill_attn_f32", "prefill_attn_bf16", "prefill_attn_f16"):
        fn = getattr(lib, name)
        fn.argtypes = [P, P, P, P] + tail
        fn.restype = I
    lib.prefill_attn_ex.argtypes = [I, P, I64, P, P, I64, P, I64, I, I, I, I, I, I, I, P, SZ, P]
    lib.prefill_attn_ex.restype = I
    lib.prefill_attn_noalloc_ex.argtypes = [I, P, I64, P, P, I64, P, I64, I, I, I, I, I, I, I, P]
    lib.prefill_attn_noalloc_ex.restype = I
    lib.prefill_attn_vmirror_ex.argtypes = [I, P, I64, P, P, I64, P, I, I, P, I64, I, I, I, I, I, I, P,
                                            SZ, P]
    lib.prefill_attn_vmirror_ex.restype = I
    lib.prefill_attn_vmirror_bytes.argtypes = [I, I, I, I]
    lib.prefill_attn_vmirror_bytes.restype = SZ
    lib.prefill_attn_ring_ex.argtypes = [I, P, I64, P, P, I64, I, P, I64, I, I, I, I, I, I, I, P, SZ,
                                         P]
    lib.prefill_attn_ring_ex.restype = I
    lib.prefill_kv_write.argtypes = [I, P, P, I64, P, P, I64, I, I, I, I, I, P]
    lib.prefill_attn_paged_ex.argtypes = [I, P, I64, P, P, I, I, P, P, I64, I, I, I, I, I, I, I, P,
                                          SZ, P]
    lib.prefill_attn_paged_ex.restype = I
    lib.prefill_attn_paged_dev_ex.argtypes = [I, P, I64, P, P, I, I, P, P, I64, I, I, P, I, I, I, I,
                                              I, P, SZ, P]
    lib.prefill_attn_paged_dev_ex.restype = I
    lib.prefill_kv_write.restype = I
    lib.prefill_attn_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.prefill_attn_workspace_bytes.restype = SZ
    lib.prefill_attn_plan.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(I64), I]
    lib.prefill_attn_plan.restype = I
    lib.prefill_attn_strerror.argtypes = [I]
    lib.prefill_attn_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/prefill_attn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prefill_\w+)\s*\(", text)))


def header_define(name: str) -> int:
    """Integer value of a #define in include/prefill_attn.h."""
    m = re.search(r"#define\s+" + re.escape(name) + r"\s+(\d+)", open(HEADER).read())
    if not m:
        raise KeyError(name)
    return int(m.group(1))


def strerror(status: int) -> str:
    try:
        return load().prefill_attn_strerror(int(status)).decode()
    except Exception:  # the library may be what failed to load
        return "unknown"


def workspace_bytes(dtype: str, T, start_pos, num_heads, num_kv_heads, head_dim, window=0) -> int:
    return int(load().prefill_attn_workspace_bytes(DTYPE_CODES[dtype], T, start_pos, num_heads,
                                                   num_kv_heads, head_dim, window))


def vmirror_bytes(dtype: str, num_kv_heads, head_dim, capacity) -> int:
    """Bytes of the V mirror prefill_attn_vmirror_ex reads (0: not needed)."""
    return int(load().prefill_attn_vmirror_bytes(DTYPE_CODES[dtype], num_kv_heads, head_dim, capacity))


def plan(dtype: str, T, start_pos, num_heads, num_kv_heads, head_dim, window=0) -> dict:
    info = (ctypes.c_int64 * 8)()
    st = load().prefill_attn_plan(DTYPE_CODES[dtype], T, start_pos, num_heads, num_kv_heads,
                                  head_dim, window, info, 8)
    if st != PA_OK:
        raise PrefillAttnError(st, "prefill_attn_plan")
    return dict(zip(PLAN_FIELDS, list(info)))


# ---- torch marshalling --------------------------------------------------------

def _dtype_of(t) -> str:
    import torch
    m = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}
    if t.dtype not in m:
        raise TypeError(f"unsupported storage type {t.dtype}")
    return m[t.dtype]


def _need(t, elems: int, what: str):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous (strides are passed explicitly)")
    if t.numel() < elems:
        raise ValueError(f"{what} holds {t.numel()} elements, the call reads/writes {elems}")


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def prefill_attn(q, k_cache, v_cache, out, T, start_pos, num_heads, num_kv_heads, head_dim,
                 window=0, stream=None):
    """Packed call: q [T, H*D], caches [KVH, L, D] (L = start_pos+T), out fp32 [T, H*D]."""
    dt = _dtype_of(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one storage type")
    import torch
    if out.dtype != torch.float32:
        raise TypeError("out must be float32")
    L = start_pos + T
    _need(q, T * num_heads * head_dim, "q")
    _need(k_cache, num_kv_heads * L * head_dim, "k_cache")
    _need(v_cache, num_kv_heads * L * head_dim, "v_cache")
    _need(out, T * num_heads * head_dim, "out")
    fn = getattr(load(), {"f32": "prefill_attn_f32", "bf16": "prefill_attn_bf16",
                          "f16": "prefill_attn_f16"}[dt])
    st = fn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), T, start_pos,
            num_heads, num_kv_heads, head_dim, window, _stream(stream))
    if st != PA_OK:
        raise PrefillAttnError(st, fn.__name__)
    return out


class PreparedCall:
    """prefill_attn_ex (prefill_attn_ring_ex when ring_slots is given, the
    paged forms with a page table, prefill_attn_vmirror_ex with a v_mirror)
    with its arguments checked and marshalled once.  out may be float32,
    bfloat16 or float16 (out_dtype follows its dtype).

    For callers that launch the same call repeatedly (a chunk loop, a
    benchmark): calling the object issues just the C-ABI call.  The tensors
    are kept referenced; their storage must not be reallocated meanwhile.
    """

    def __init__(self, q, q_row_stride, k_cache, v_cache, kv_head_stride, out, out_row_stride, T,
                 start_pos, num_heads, num_kv_heads, head_dim, window=0, workspace=None,
                 stream=None, ring_slots=None, page_table=None, page_size=None,
                 start_pos_dev=None, v_mirror=None, mirror_capacity=None, mirror_keys=0):
        dt = _dtype_of(q)
        if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
            raise TypeError("q, k_cache and v_cache must share one storage type")
        rows = start_pos + T if ring_slots is None else ring_slots
        _need(q, (T - 1) * q_row_stride + num_heads * head_dim, "q")
        if page_table is None:
            _need(k_cache, (num_kv_heads - 1) * kv_head_stride + rows * head_dim, "k_cache")
            _need(v_cache, (num_kv_heads - 1) * kv_head_stride + rows * head_dim, "v_cache")
        else:
            # pools of whole pages; the table covers the call's keys
            page_elems = page_size * num_kv_heads * head_dim
            _need(k_cache, page_elems, "k_pool")
            _need(v_cache, k_cache.numel(), "v_pool")
            import torch
            if page_table.dtype != torch.int32:
                raise TypeError("page_table must be int32")
            _need(page_table, -(-(start_pos + T) // page_size), "page_table")
        _need(out, (T - 1) * out_row_stride + num_heads * head_dim, "out")
        out_dt = DTYPE_CODES[_dtype_of(out)]
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        head = (DTYPE_CODES[dt], q.data_ptr(), q_row_stride, k_cache.data_ptr(),
                v_cache.data_ptr(), kv_head_stride)
        tail = (out.data_ptr(), out_row_stride, out_dt, T, start_pos, num_heads, num_kv_heads,
                head_dim, window, ws_ptr, ws_bytes, _stream(stream))
        if v_mirror is not None:
            if ring_slots is not None or page_table is not None or window != 0:
                raise ValueError("the V mirror serves linear caches without a window")
            if not v_mirror.is_cuda or not v_mirror.is_contiguous():
                raise ValueError("v_mirror must be a contiguous device tensor")
            nb = vmirror_bytes(dt, num_kv_heads, head_dim, mirror_capacity)
            if v_mirror.numel() * v_mirror.element_size() < nb:
                raise ValueError(f"v_mirror holds {v_mirror.numel() * v_mirror.element_size()} bytes, "
                                 f"the call needs {nb}")
            self._name, self._fn = "prefill_attn_vmirror_ex", load().prefill_attn_vmirror_ex
            self._args = head + (v_mirror.data_ptr(), int(mirror_capacity), int(mirror_keys)) + \
                (out.data_ptr(), out_row_stride, out_dt, T, start_pos, num_heads, num_kv_heads,
                 head_dim, ws_ptr, ws_bytes, _stream(stream))
        elif start_pos_dev is not None:
            # start_pos is the largest the device value may take
            import torch
            if page_table is None or start_pos_dev.dtype != torch.int32:
                raise TypeError("start_pos_dev needs a paged cache and an int32 device tensor")
            _need(start_pos_dev, 1, "start_pos_dev")
            self._name, self._fn = "prefill_attn_paged_dev_ex", load().prefill_attn_paged_dev_ex
            self._args = (DTYPE_CODES[dt], q.data_ptr(), q_row_stride, k_cache.data_ptr(),
                          v_cache.data_ptr(), int(page_size),
                          k_cache.numel() // (page_size * num_kv_heads * head_dim),
                          page_table.data_ptr(), out.data_ptr(), out_row_stride, out_dt, T,
                          start_pos_dev.data_ptr(), start_pos, num_heads, num_kv_heads, head_dim,
                          window, ws_ptr, ws_bytes, _stream(stream))
        elif page_table is not None:
            self._name, self._fn = "prefill_attn_paged_ex", load().prefill_attn_paged_ex
            self._args = (DTYPE_CODES[dt], q.data_ptr(), q_row_stride, k_cache.data_ptr(),
                          v_cache.data_ptr(), int(page_size),
                          k_cache.numel() // (page_size * num_kv_heads * head_dim),
                          page_table.data_ptr()) + tail
        elif ring_slots is None:
            self._name, self._fn, self._args = "prefill_attn_ex", load().prefill_attn_ex, head + tail
        else:
            self._name, self._fn = "prefill_attn_ring_ex", load().prefill_attn_ring_ex
            self._args = head + (int(ring_slots),) + tail
        self._keep = (q, k_cache, v_cache, out, workspace, page_table, start_pos_dev, v_mirror)
        self.out = out

    def __call__(self):
        st = self._fn(*self._args)
        if st != PA_OK:
            raise PrefillAttnError(st, self._name)
        return self.out


def prefill_attn_ex(q, q_row_stride, k_cache, v_cache, kv_head_stride, out, out_row_stride, T,
                    start_pos, num_heads, num_kv_heads, head_dim, window=0, workspace=None,
                    stream=None):
    """Strided call; workspace is a device tensor (any dtype) or None; out is
    float32, bfloat16 or float16."""
    return PreparedCall(q, q_row_stride, k_cache, v_cache, kv_head_stride, out, out_row_stride, T,
                        start_pos, num_heads, num_kv_heads, head_dim, window, workspace, stream)()


def prefill_attn_noalloc_ex(q, q_row_stride, k_cache, v_cache, kv_head_stride, out, out_row_stride,
                            T, start_pos, num_heads, num_kv_heads, head_dim, window=0, stream=None):
    """prefill_attn_ex without a workspace: the library's fixed per-GPU scratch
    array serves instead, and nothing is allocated.  Calls that overlap in
    time on one GPU must not be issued (they share the array)."""
    dt = _dtype_of(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one storage type")
    L = start_pos + T
    _need(q, (T - 1) * q_row_stride + num_heads * head_dim, "q")
    _need(k_cache, (num_kv_heads - 1) * kv_head_stride + L * head_dim, "k_cache")
    _need(v_cache, (num_kv_heads - 1) * kv_head_stride + L * head_dim, "v_cache")
    _need(out, (T - 1) * out_row_stride + num_heads * head_dim, "out")
    st = load().prefill_attn_noalloc_ex(DTYPE_CODES[dt], q.data_ptr(), q_row_stride, k_cache.data_ptr(),
                                        v_cache.data_ptr(), kv_head_stride, out.data_ptr(), out_row_stride,
                                        DTYPE_CODES[_dtype_of(out)], T, start_pos, num_heads, num_kv_heads,
                                        head_dim, window, _stream(stream))
    if st != PA_OK:
        raise PrefillAttnError(st, "prefill_attn_noalloc_ex")
    return out


def prefill_attn_vmirror_ex(q, q_row_stride, k_cache, v_cache, kv_head_stride, v_mirror,
                            mirror_capacity, mirror_keys, out, out_row_stride, T, start_pos, num_heads,
                            num_kv_heads, head_dim, workspace=None, stream=None):
    """Causal call (no window) that keeps V's operand-order copy in v_mirror
    (a device tensor of vmirror_bytes(...) bytes) across the chunks of a
    sequence: keys 0 .. mirror_keys-1 are already in it, the call adds the
    rest up to start_pos+T."""
    return PreparedCall(q, q_row_stride, k_cache, v_cache, kv_head_stride, out, out_row_stride, T,
                        start_pos, num_heads, num_kv_heads, head_dim, 0, workspace, stream,
                        v_mirror=v_mirror, mirror_capacity=mirror_capacity, mirror_keys=mirror_keys)()


def prefill_attn_ring_ex(q, q_row_stride, k_ring, v_ring, kv_head_stride, ring_slots, out,
                         out_row_stride, T, start_pos, num_heads, num_kv_heads, head_dim, window=0,
                         workspace=None, stream=None):
    """Strided call over a ring cache: key j in slot j % ring_slots of each kv head."""
    return PreparedCall(q, q_row_stride, k_ring, v_ring, kv_head_stride, out, out_row_stride, T,
                        start_pos, num_heads, num_kv_heads, head_dim, window, workspace, stream,
                        ring_slots=ring_slots)()


def prefill_attn_paged_ex(q, q_row_stride, k_pool, v_pool, page_size, page_table, out,
                          out_row_stride, T, start_pos, num_heads, num_kv_heads, head_dim, window=0,
                          workspace=None, stream=None):
    """Strided call over a paged cache: pools of pages of page_size positions of
    every kv head (num_pages = pool elements / (page_size*num_kv_heads*head_dim)),
    key j in page page_table[j // page_size] (int32 device tensor)."""
    return PreparedCall(q, q_row_stride, k_pool, v_pool, 0, out, out_row_stride, T, start_pos,
                        num_heads, num_kv_heads, head_dim, window, workspace, stream,
                        page_table=page_table, page_size=page_size)()


def prefill_kv_write(k_src, v_src, src_row_stride, k_cache, v_cache, kv_head_stride, T, start_pos,
                     num_kv_heads, head_dim, ring_slots=0, stream=None):
    """Store the chunk's K/V rows in the cache: row start_pos + i, or slot
    (start_pos + i) % ring_slots of a ring (ring_slots > 0)."""
    dt = _dtype_of(k_src)
    for t in (v_src, k_cache, v_cache):
        if t.dtype != k_src.dtype:
            raise TypeError("sources and caches must share one storage type")
    rows = ring_slots if ring_slots else start_pos + T
    _need(k_src, (T - 1) * src_row_stride + num_kv_heads * head_dim, "k_src")
    _need(v_src, (T - 1) * src_row_stride + num_kv_heads * head_dim, "v_src")
    _need(k_cache, (num_kv_heads - 1) * kv_head_stride + rows * head_dim, "k_cache")
    _need(v_cache, (num_kv_heads - 1) * kv_head_stride + rows * head_dim, "v_cache")
    st = load().prefill_kv_write(DTYPE_CODES[dt], k_src.data_ptr(), v_src.data_ptr(), src_row_stride,
                                 k_cache.data_ptr(), v_cache.data_ptr(), kv_head_stride,
                                 int(ring_slots), T, start_pos, num_kv_heads, head_dim,
                                 _stream(stream))
    if st != PA_OK:
        raise PrefillAttnError(st, "prefill_kv_write")
