"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments before anything is enqueued."""
import ctypes

import pytest

import causal_gqa_attention_prefill_amd as pa
from causal_gqa_attention_prefill_amd import binding

FAKE = 0x10000  # a non-null, 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    return pa.load()


def test_exports_every_declared_function(lib):
    names = pa.header_functions()
    assert set(names) == {"prefill_attn_f32", "prefill_attn_bf16", "prefill_attn_f16",
                          "prefill_attn_ex", "prefill_attn_ring_ex", "prefill_attn_workspace_bytes",
                          "prefill_attn_plan", "prefill_attn_strerror", "prefill_kv_write",
                          "prefill_attn_paged_ex", "prefill_attn_paged_dev_ex", "prefill_attn_noalloc_ex",
                          "prefill_attn_vmirror_ex", "prefill_attn_vmirror_bytes"}
    for n in names:
        assert hasattr(lib, n), n


def _header_signatures():
    """{name: [parameter declarations]} of the functions the header declares."""
    import re
    text = open(binding.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    sigs = {}
    for name, params in re.findall(r"\b(prefill_\w+)\s*\(([^)]*)\)\s*;", text):
        sigs[name] = [p.strip() for p in params.split(",") if p.strip() and p.strip() != "void"]
    return sigs


def test_binding_matches_header_signatures(lib):
    """Every declared function is bound with as many arguments as the header
    gives it, and each pointer, 64-bit and size_t parameter has a matching
    ctypes type (a parameter added to the ABI but not to the binding fails here)."""
    sigs = _header_signatures()
    assert set(sigs) == set(pa.header_functions())
    for name, params in sigs.items():
        argtypes = getattr(lib, name).argtypes
        assert argtypes is not None and len(argtypes) == len(params), (name, params, argtypes)
        for decl, ct in zip(params, argtypes):
            if "*" in decl:
                assert ct in (ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)), (name, decl, ct)
            elif decl.startswith("int64_t"):
                assert ct is ctypes.c_int64, (name, decl, ct)
            elif decl.startswith("size_t"):
                assert ct is ctypes.c_size_t, (name, decl, ct)
            else:
                assert decl.startswith("int ") and ct is ctypes.c_int, (name, decl, ct)


def test_strerror(lib):
    for code in range(5):
        assert pa.strerror(code) not in ("", "unknown status")
    assert pa.strerror(99) == "unknown status"


def _packed(lib, fn, q=FAKE, k=FAKE, v=FAKE, out=FAKE, T=4, sp=0, H=4, KVH=2, D=64, W=0):
    return getattr(lib, fn)(q, k, v, out, T, sp, H, KVH, D, W, None)


@pytest.mark.parametrize("fn", ["prefill_attn_f32", "prefill_attn_bf16", "prefill_attn_f16"])
def test_invalid_arguments(lib, fn):
    E = pa.PA_ERR_INVALID_ARG
    assert _packed(lib, fn, q=None) == E
    assert _packed(lib, fn, k=None) == E
    assert _packed(lib, fn, v=None) == E
    assert _packed(lib, fn, out=None) == E
    assert _packed(lib, fn, T=0) == E
    assert _packed(lib, fn, T=-3) == E
    assert _packed(lib, fn, sp=-1) == E
    assert _packed(lib, fn, H=0) == E
    assert _packed(lib, fn, KVH=0) == E
    assert _packed(lib, fn, H=6, KVH=4) == E
    assert _packed(lib, fn, W=-1) == E
    assert _packed(lib, fn, T=2**30, sp=2**30 + 5) == E


@pytest.mark.parametrize("fn", ["prefill_attn_f32", "prefill_attn_bf16", "prefill_attn_f16"])
def test_unsupported(lib, fn):
    U = pa.PA_ERR_UNSUPPORTED
    for D in (16, 48, 100, 1024):
        assert _packed(lib, fn, D=D) == U
    assert _packed(lib, fn, H=256, KVH=1) == U       # group larger than a work-group's rows
    assert _packed(lib, fn, q=FAKE + 4) == U          # misaligned
    if fn == "prefill_attn_f32":
        assert _packed(lib, fn, D=512) == U


def test_ex_strides_and_workspace(lib):
    ex = lib.prefill_attn_ex
    # strides below their minimum
    assert ex(1, FAKE, 100, FAKE, FAKE, 64 * 10, FAKE, 128, 0, 4, 6, 2, 2, 64, 0, None, 0, None) == 1
    assert ex(1, FAKE, 128, FAKE, FAKE, 64 * 9, FAKE, 128, 0, 4, 6, 2, 2, 64, 0, None, 0, None) == 1
    assert ex(1, FAKE, 128, FAKE, FAKE, 64 * 10, FAKE, 127, 0, 4, 6, 2, 2, 64, 0, None, 0, None) == 1
    # unknown dtype, unknown output dtype
    assert ex(7, FAKE, 128, FAKE, FAKE, 640, FAKE, 128, 0, 4, 6, 2, 2, 64, 0, None, 0, None) == 2
    assert ex(1, FAKE, 128, FAKE, FAKE, 640, FAKE, 128, 3, 4, 6, 2, 2, 64, 0, None, 0, None) == 2
    assert ex(1, FAKE, 128, FAKE, FAKE, 640, FAKE, 128, -1, 4, 6, 2, 2, 64, 0, None, 0, None) == 2
    # a row stride that breaks 16-byte alignment of rows
    assert ex(1, FAKE, 132, FAKE, FAKE, 640, FAKE, 128, 0, 4, 6, 2, 2, 64, 0, None, 0, None) == 2
    # an output row stride that is not a multiple of 4 elements, for any output type
    for od in (0, 1, 2):
        assert ex(1, FAKE, 128, FAKE, FAKE, 640, FAKE, 130, od, 4, 6, 2, 2, 64, 0, None, 0, None) == 2
    # a split plan without (or with too little) workspace
    need = pa.workspace_bytes("bf16", 64, 8000, 8, 8, 128)
    assert need > 0
    args = (1, FAKE, 8 * 128, FAKE, FAKE, 8064 * 128, FAKE, 8 * 128, 1, 64, 8000, 8, 8, 128, 0)
    assert ex(*args, None, 0, None) == pa.PA_ERR_WORKSPACE
    assert ex(*args, FAKE, need - 1, None) == pa.PA_ERR_WORKSPACE
    assert ex(*args, FAKE + 16, need, None) == pa.PA_ERR_WORKSPACE   # not 256-byte aligned


def test_head_size_limit(lib):
    """The 16-bit kernels address one kv head's rows with 32-bit buffer
    offsets: a cache with one row per head more than 0x7FE00000 bytes hold is
    refused before anything is enqueued (fp32 caches are addressed in 64 bits)."""
    D = 128
    rows = 0x7FE00000 // (D * 2)
    L = rows + 1
    for dtype in (1, 2):
        assert lib.prefill_attn_ex(dtype, FAKE, 4 * D, FAKE, FAKE, L * D, FAKE, 4 * D, 0, 64, L - 64, 4,
                                   1, D, 0, None, 0, None) == pa.PA_ERR_UNSUPPORTED
    # the same shape in fp32 passes the shape checks (here it stops at the workspace)
    assert lib.prefill_attn_ex(0, FAKE, 4 * D, FAKE, FAKE, L * D, FAKE, 4 * D, 0, 64, L - 64, 4,
                               1, D, 0, None, 0, None) == pa.PA_ERR_WORKSPACE


def test_plan_shapes():
    p = pa.plan("bf16", 2048, 6144, 32, 8, 128)
    assert p["tokens_per_tile"] * 4 == 128 and p["query_tiles"] == 64
    # a full causal grid without a window pairs the long and the short query
    # tile of each kv head in one eight-wavefront work-group
    assert p["kv_splits"] == 1 and p["waves_per_workgroup"] == 8 and p["workgroups"] == 32 * 8
    # a window (or a grid that leaves CUs idle) keeps one query tile per work-group
    pw = pa.plan("bf16", 2048, 6144, 32, 8, 128, 1000)
    assert pw["workgroups"] == 64 * 8 * pw["kv_splits"] and pw["waves_per_workgroup"] == 4
    ps = pa.plan("bf16", 256, 0, 32, 8, 128)
    assert ps["workgroups"] == 8 * 8 * ps["kv_splits"] and ps["waves_per_workgroup"] == 4
    # more pairs than CUs (a second round): single tiles, refilled by the dispatcher
    for T in (8192, 2080):
        pl = pa.plan("bf16", T, 0, 32, 8, 128)
        assert pl["waves_per_workgroup"] == 4 and pl["workgroups"] == pl["query_tiles"] * 8
    # every (tile, kv head) visits only KV tiles that hold a valid key of one of its rows
    bk = p["keys_per_tile"]
    tiles = 0
    for qt in range(64):
        lo_pos, hi_pos = 6144 + 32 * qt, 6144 + 32 * qt + 31
        tiles += hi_pos // bk - 0 // bk + 1
    assert p["kv_tiles_visited"] == tiles * 8
    # the window keeps a tile's KV range to ~window + tile keys
    w = pa.plan("bf16", 2048, 129024, 8, 4, 256, 1024)
    per_tile = w["kv_tiles_visited"] / (w["query_tiles"] * 4)
    assert per_tile <= (1024 + w["tokens_per_tile"]) / w["keys_per_tile"] + 2
    assert pa.workspace_bytes("bf16", 2048, 6144, 32, 8, 128) == p["workspace_bytes"]
    with pytest.raises(pa.PrefillAttnError):
        pa.plan("bf16", 4, 0, 6, 4, 64)


def test_binding_has_no_cpu_path():
    src = open(binding.__file__).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "numpy" not in src


def test_prepared_call_rejects_host_tensors():
    # the prepared form checks its arguments like prefill_attn_ex: host tensors are refused
    import torch
    q = torch.zeros(4, 2 * 32, dtype=torch.bfloat16)
    kv = torch.zeros(1, 4, 32, dtype=torch.bfloat16)
    out = torch.zeros(4, 2 * 32, dtype=torch.float32)
    with pytest.raises(ValueError):
        pa.PreparedCall(q, 64, kv, kv, 4 * 32, out, 64, 4, 0, 2, 1, 32)
    with pytest.raises(ValueError):
        pa.prefill_attn_ex(q, 64, kv, kv, 4 * 32, out, 64, 4, 0, 2, 1, 32)


def test_ring_arguments(lib):
    """The ring form refuses rings that cannot hold every key the chunk reads,
    a head stride below ring_slots*head_dim and a non-positive slot count,
    before anything is enqueued (fake device pointers are never touched)."""
    rx = lib.prefill_attn_ring_ex
    E, U = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED
    H, KVH, D, T, sp, W = 8, 4, 256, 64, 5000, 100

    def call(ring, kvs=None, w=W, t=T, s=sp, dtype=1):
        kvs = ring * D if kvs is None else kvs
        return rx(dtype, FAKE, H * D, FAKE, FAKE, kvs, ring, FAKE, H * D, 0, t, s, H, KVH, D, w,
                  None, 0, None)

    assert call(0) == E
    assert call(-5) == E
    assert call(W + T - 2) == E                    # one slot short of window + T - 1
    assert call(W + T - 1, kvs=(W + T - 1) * D - 8) == E
    assert call(3000, w=0) == E                    # no window: the ring must hold all L keys
    assert call(W + T - 1, dtype=7) == U
    # a ring too large for 32-bit buffer offsets of the 16-bit kernels
    assert call(2 ** 22, w=0, s=2 ** 22 - T) == U
    # every shape check of prefill_attn_ex applies too
    assert call(W + T - 1, t=0) == E


def test_kv_write_arguments(lib):
    """prefill_kv_write checks its arguments before anything is enqueued."""
    kw = lib.prefill_kv_write
    E, U = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED
    KVH, D, T, sp = 2, 64, 10, 100

    def call(dtype=1, ks=FAKE, vs=FAKE, srs=KVH * D, kc=FAKE, vc=FAKE, kvs=None, ring=0, t=T, s=sp,
             kvh=KVH, d=D):
        kvs = ((ring or (s + t)) * d) if kvs is None else kvs
        return kw(dtype, ks, vs, srs, kc, vc, kvs, ring, t, s, kvh, d, None)

    assert call(ks=None) == E and call(vc=None) == E
    assert call(t=0) == E and call(s=-1) == E and call(kvh=0) == E and call(ring=-1) == E
    assert call(srs=KVH * D - 1) == E
    assert call(kvs=(sp + T) * D - 8) == E
    assert call(ring=16, kvs=16 * D - 8) == E
    assert call(dtype=9) == U
    assert call(d=4) == U                      # 8-byte rows
    assert call(ks=FAKE + 8) == U              # misaligned
    assert call(srs=KVH * D + 4) == U          # source rows not 16-byte multiples


def test_paged_arguments(lib):
    """prefill_attn_paged_ex refuses bad page sizes, a missing table or pool
    size, and every bad shape prefill_attn_ex refuses, before enqueuing."""
    px = lib.prefill_attn_paged_ex
    E, U = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED
    H, KVH, D = 8, 2, 128

    def call(P=256, npages=10, table=FAKE, T=4, sp=1000, w=0, dtype=1, q=FAKE, od=0):
        return px(dtype, q, H * D, FAKE, FAKE, P, npages, table, FAKE, H * D, od, T, sp, H, KVH, D, w,
                  None, 0, None)

    assert call(table=None) == E
    assert call(npages=0) == E
    assert call(P=32) == U and call(P=96) == U and call(P=0) == U
    assert call(T=0) == E and call(sp=-1) == E and call(w=-2) == E
    assert call(q=None) == E
    assert call(dtype=5) == U
    assert call(q=FAKE + 2) == U
    assert call(od=4) == U


def test_paged_dev_arguments(lib):
    """The device-start form needs its start buffer and checks the rest as the
    paged form does, for the largest start_pos."""
    px = lib.prefill_attn_paged_dev_ex
    E, U = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED
    H, KVH, D = 8, 2, 128

    def call(sp_dev=FAKE, maxsp=1000, P=256, table=FAKE, T=4):
        return px(1, FAKE, H * D, FAKE, FAKE, P, 10, table, FAKE, H * D, 0, T, sp_dev, maxsp, H, KVH,
                  D, 0, None, 0, None)

    assert call(sp_dev=None) == E
    assert call(table=None) == E
    assert call(maxsp=-1) == E
    assert call(T=0) == E
    assert call(P=48) == U


def test_noalloc_arguments(lib):
    """The no-allocation form checks its arguments like prefill_attn_ex,
    before it looks up its scratch (so nothing here touches a GPU)."""
    E, U = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED
    fn = lib.prefill_attn_noalloc_ex

    def call(q=FAKE, qs=256, k=FAKE, v=FAKE, kvs=64 * 64, out=FAKE, os_=256, odt=0, T=4, sp=60, H=4,
             KVH=2, D=64, W=0, dt=pa.PA_DTYPE_BF16):
        return fn(dt, q, qs, k, v, kvs, out, os_, odt, T, sp, H, KVH, D, W, None)

    assert call(q=None) == E and call(k=None) == E and call(v=None) == E and call(out=None) == E
    assert call(T=0) == E and call(sp=-1) == E and call(W=-1) == E and call(H=6, KVH=4) == E
    assert call(qs=255) == E                 # q row shorter than H * D
    assert call(kvs=63 * 64) == E            # kv-head stride below L * D
    assert call(os_=200) == E
    assert call(D=48) == U and call(dt=7) == U and call(odt=9) == U
    assert call(q=FAKE + 8) == U             # misaligned
    assert pa.header_define("PA_NOALLOC_SCRATCH_BYTES") == 32 << 20


def test_vmirror_arguments(lib):
    """The V-mirror form checks its arguments before anything is enqueued
    (nothing here touches a GPU); the mirror's size follows its tiles."""
    E, U = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED
    fn = lib.prefill_attn_vmirror_ex
    BF = pa.PA_DTYPE_BF16

    def call(q=FAKE, qs=4 * 512, k=FAKE, v=FAKE, kvs=64 * 512, mir=FAKE, cap=64, mk=0, out=FAKE,
             os_=4 * 512, odt=0, T=4, sp=60, H=4, KVH=2, D=512, dt=BF):
        return fn(dt, q, qs, k, v, kvs, mir, cap, mk, out, os_, odt, T, sp, H, KVH, D, None, 0, None)

    assert call(q=None) == E and call(k=None) == E and call(out=None) == E
    assert call(T=0) == E and call(sp=-1) == E and call(H=6, KVH=4) == E
    assert call(kvs=63 * 512) == E            # kv-head stride below L * D
    assert call(mir=None) == E                # a mirror is needed at head_dim 512
    assert call(cap=63) == E                  # capacity below L
    assert call(mk=-1) == E and call(mk=65) == E
    assert call(mir=FAKE + 8) == U            # misaligned mirror
    assert call(D=48) == U and call(dt=7) == U
    # sizes: whole 32-key tiles of 512 bf16 values per kv head
    assert pa.vmirror_bytes("bf16", 2, 512, 64) == 2 * 64 * 512 * 2
    assert pa.vmirror_bytes("f16", 2, 512, 65) == 2 * 96 * 512 * 2
    assert pa.vmirror_bytes("bf16", 2, 128, 64) == 0      # read in place: no mirror
    assert pa.vmirror_bytes("f32", 2, 512, 64) == 0
    assert pa.vmirror_bytes("bf16", 0, 512, 64) == 0 and pa.vmirror_bytes("bf16", 2, 512, 0) == 0
    assert pa.vmirror_bytes("bf16", 1, 512, 3 << 20) == 0  # one head's share would pass 2 GiB
