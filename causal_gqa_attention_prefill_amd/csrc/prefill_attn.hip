// prefill_attn.hip -- fused chunked causal grouped-query prefill attention
// for MI355X (gfx950 / CDNA4), behind the C ABI of include/prefill_attn.h.
//
// The computation is the one of the gnosis handoff page "Prefill attention ->
// GPU: handoff", section "GPU design (the real fix)": scores = Q K^T scaled by
// 1/sqrt(head_dim), causal mask (key j valid iff j <= start_pos + t), row
// softmax, times V, with query head h reading kv head h / (H / KVH).  The
// window band is the per-row contiguous [lo, pos] band of the TensorSharp page
// "Design: closing the Gemma-4 long-prompt prefill gap", section 5 (Option A),
// read as lo = pos - window + 1.
//
// That page's plan materialises the [heads x Tq x L] scores between two
// strided-batched GEMMs and a softmax kernel, and its "Implementation status"
// lists merging the softmax into the A.V product as a follow-up.  Here everything
// is one pass over the keys (online softmax), so scores never leave
// registers:
//
//   work-group  = 4 wavefronts = 128 (token, head) rows of one GQA group:
//                 row r -> token t0 + r / G, head kvh*G + r % G, so the G
//                 query heads that share kv head kvh share every K/V tile
//                 (at head_dim 128 on a full causal grid: 8 wavefronts, the
//                 long and the short query tile of the kv head, which share
//                 the K/V tiles of their common key prefix)
//   per KV tile of BK keys (only tiles that intersect some row's band):
//     global -> LDS: K and V tiles as [key][d] (DMA, no register staging);
//                   V is read back transposed (or, at head_dim 512, from a
//                   per-call copy in MFMA operand order)
//     S^T = K Q^T   on MFMA (32x32 tiles, keys on M, rows on N); Q stays in
//                   registers for the whole loop, pre-scaled by
//                   log2(e)/sqrt(head_dim), and each chain starts at minus
//                   the row's reference max, so scores come out as exponents
//     mask          only on tiles that cut some row's band (index compares)
//     online softmax in fp32: each lane holds one row's scores for 16 keys
//                   per 32-key block, so the row max needs one exchange
//                   between the two lane halves and the row sum none
//     O^T += V^T P^T on MFMA: the S^T accumulator registers are already in
//                   the layout of the B operand, so P never goes through LDS;
//                   O^T columns are rows, so the rescale by alpha is per lane
//   epilogue    out = O / l (fp32), or per-split partials (O, m, l) that a
//               second kernel merges when the grid is split along the keys
//
// bf16/fp16 inputs use v_mfma_f32_32x32x16_{bf16,f16} (P rounded to the input
// type); fp32 inputs use v_mfma_f32_32x32x2_f32 with P kept in fp32.
//
// Correctness of the MFMA operand plumbing rests only on the accumulator
// layout (lane l, register r of a 32x32 tile holds row 8*(r/4) + 4*(l/32) +
// r%4, column l%32) and on A and B sharing the same lane/element -> k map.
// Each contraction (over head_dim for S, over keys for O) pairs A's and B's
// element (l/32, e) with the same index, whatever index the hardware assigns
// to that slot.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <type_traits>
#include <mutex>
#include <vector>

#include "prefill_attn.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
constexpr int kXcds = 8;          // MI355X: 8 accelerator dies, work-groups dealt round-robin
constexpr int kCus = 256;         // MI355X compute units

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Params {
    const void *q;
    const void *k;
    const void *v;
    void *out;        // [T] rows of out_row_stride elements of out_dtype
    int out_dtype;    // PA_DTYPE_F32, or BF16 / F16 (rounded to nearest even)
    float *ws_o;      // [S][T*H][D] split partials, normalised by their own l
    float2 *ws_ml;    // [S][T*H]    (running max of raw scores, l)
    int64_t q_row_stride, kv_head_stride, out_row_stride;
    int T, start_pos, H, KVH, G, window;
    int TQ;           // query tokens per tile
    int nq;           // query tiles
    int S;            // key splits per tile
    int n_items;      // nq * KVH * S work-groups
    float c;          // log2(e) / sqrt(head_dim)
    int order;        // 1: within a die, longest query tiles first then shortest first; 0: longest first
    int pair;         // 1: each work-group holds two query tiles of one kv head (8 wavefronts)
    int kv_bytes;     // bytes of the L valid rows (linear) or of the ring slots of one kv head
    int L;            // keys of the call: start_pos + T
    int ring;         // ring cache: key j sits in slot j % ring of its kv head; 0: row j
    const int32_t *page_table;  // paged cache: page of each block of 2^page_shift keys (else null)
    int page_shift, num_pages;
    const int32_t *start_pos_dev;  // device-side start_pos (at most start_pos), else null
    const uint16_t *vop;   // V of the call's KV tiles in MFMA operand order (16-bit kernels)
    int vop_kt_lo;         // first KV tile held in vop
    int vop_tiles;         // KV tiles per kv head held in vop
    int vop_pack0;         // first tile of vop (from vop_kt_lo) the pass rewrites this call
};

// A call whose start_pos sits in device memory (so that one captured graph
// serves every length): the plan was made for the largest start_pos, passed
// in p.start_pos; the work-groups take the current one.
__device__ inline void take_device_start(Params &p) {
    if (p.start_pos_dev) {
        p.start_pos = min(max(*p.start_pos_dev, 0), p.start_pos);
        p.L = p.start_pos + p.T;
    }
}

// K/V cache layouts: key j of kv head kh is row j of the head's block
// (linear), slot j % ring of it (ring, sliding-window layers), or row
// j % page_size of page page_table[j / page_size] of a pool shared by the
// kv heads (paged): element (pg, kh, r, d) at pool[((pg*KVH + kh)*page_size + r)*D + d].
constexpr int kLinear = 0, kRing = 1, kPaged = 2;

// Element offset of row (kh, key j) of a cache in any layout, or -1 when a
// paged cache's entry for j lies outside the pool (such rows read as zero).
template <int D>
__device__ inline int64_t kv_row(const Params &p, int kh, int j) {
    if (p.page_table) {
        const int pg = p.page_table[j >> p.page_shift];
        if (pg < 0 || pg >= p.num_pages) return -1;
        return ((((int64_t)pg * p.KVH + kh) << p.page_shift) + (j & ((1 << p.page_shift) - 1))) * D;
    }
    return (int64_t)kh * p.kv_head_stride + (int64_t)(p.ring ? j % p.ring : j) * D;
}

// ---- storage types ---------------------------------------------------------

struct Bf16 {
    __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack(float lo, float hi) {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    // both halves times c, rounded to nearest even
    __device__ static inline uint32_t scale2(uint32_t x, float c) {
        const bf16x2 v = __builtin_bit_cast(bf16x2, x);
        return pack((float)v[0] * c, (float)v[1] * c);
    }
};

struct F16 {
    __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack(float lo, float hi) {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ static inline uint32_t scale2(uint32_t x, float c) {
        const f16x2 v = __builtin_bit_cast(f16x2, x);
        return pack((float)v[0] * c, (float)v[1] * c);
    }
};

// Four consecutive outputs of one row at element e of out: fp32 (ODT
// PA_DTYPE_F32), or rounded to the nearest even bf16 / fp16.  Written once and
// not read again by the call: non-temporal stores keep them from displacing
// cached K/V lines.
template <int ODT>
__device__ inline void store_out4(void *out, int64_t e, f32x4 v) {
    if constexpr (ODT == PA_DTYPE_F32) {
        __builtin_nontemporal_store(v, (f32x4 *)((float *)out + e));
    } else {
        const u32x2 x = ODT == PA_DTYPE_BF16
                            ? u32x2{Bf16::pack(v[0], v[1]), Bf16::pack(v[2], v[3])}
                            : u32x2{F16::pack(v[0], v[1]), F16::pack(v[2], v[3])};
        __builtin_nontemporal_store(x, (u32x2 *)((uint16_t *)out + e));
    }
}

// f(std::integral_constant<int, out_dtype>) for the call's output type, so
// that a row's stores are one branch-free run of the type's instructions.
template <class F>
__device__ inline void with_out_dtype(int out_dtype, F &&f) {
    if (out_dtype == PA_DTYPE_BF16)
        f(std::integral_constant<int, PA_DTYPE_BF16>{});
    else if (out_dtype == PA_DTYPE_F16)
        f(std::integral_constant<int, PA_DTYPE_F16>{});
    else
        f(std::integral_constant<int, PA_DTYPE_F32>{});
}

// ---- work-group -> (query tile, kv head, split) ----------------------------

// Work-group b runs on die b % 8.  Give each die a contiguous range of
// logical items so that the tiles of one kv head (and one key split) share a
// die's L2; inside a range the query tile varies fastest.
__device__ inline int xcd_logical_item(int b, int n) {
    const int xcd = b % kXcds, slot = b / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    return xcd * per + min(xcd, rem) + slot;
}

__device__ inline int first_key(int pos, int window) {
    return (window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;
}

struct Tile {
    int kvh, split, t0, t_last;
    int kt_begin, kt_end;          // this work-group's KV tiles [begin, end)
    // Keys the work-group's rows read: [klo, kend), from the first row's
    // window start to the last row's position.  The other rows of its first
    // and last KV tile are loaded as zeros (their keys are valid for no row
    // here), so whatever the cache holds there cannot reach the output
    // through a product with probability 0.
    int klo, kend;
};

template <int BK>
__device__ inline Tile locate(const Params &p) {
    Tile w;
    const int item = xcd_logical_item(blockIdx.x, p.n_items);
    const int qi = item % p.nq;
    const int rest = item / p.nq;
    w.split = rest % p.S;
    w.kvh = rest / p.S;
    // order 1 (two resident work-groups per CU): the first half of a die's
    // range runs the longest rows first and the second half the shortest
    // first, so the two work-groups a CU receives when the range is dealt
    // round-robin over its CUs carry similar work.  order 0 (one per CU):
    // longest first, so that the dispatcher's refills balance the tail.
    const int half_ = (p.nq + 1) / 2;
    const int qtile = p.order == 0 ? p.nq - 1 - qi : qi < half_ ? p.nq - 1 - qi : qi - half_;
    w.t0 = qtile * p.TQ;
    w.t_last = min(w.t0 + p.TQ, p.T) - 1;
    const int lo = first_key(p.start_pos + w.t0, p.window);
    const int hi = p.start_pos + w.t_last;
    const int kb = lo / BK, ke = hi / BK + 1;
    const int per = (ke - kb + p.S - 1) / p.S;
    w.kt_begin = min(ke, kb + w.split * per);
    w.kt_end = min(ke, w.kt_begin + per);
    w.klo = lo;
    w.kend = hi + 1;
    return w;
}

// Paired work-groups (causal, no window, no key split, an even number of
// query tiles; the host plans pairs only then): item -> (kv head, j);
// wavefronts 0..3 take the long query tile nq-1-j, wavefronts 4..7 the short
// one j.  The short tile's keys are a prefix of the long one's, so the
// work-group steps through the long tile's KV range and every tile both need
// comes into LDS once instead of once per work-group; the short tile's
// wavefronts skip the tiles past their rows.  Returns the group's tile; kb/ke
// get the work-group's KV range.
template <int BK>
__device__ inline Tile locate_pair(const Params &p, int grp, int &kb, int &ke) {
    const int item = xcd_logical_item(blockIdx.x, p.n_items);
    const int np = p.nq / 2;
    const int j = item % np, kvh = item / np;
    const int ql = p.nq - 1 - j, qs = j;
    const int tl0 = ql * p.TQ, tl1 = min(tl0 + p.TQ, p.T) - 1;
    const int ts0 = qs * p.TQ, ts1 = min(ts0 + p.TQ, p.T) - 1;
    // union of the two key ranges: the short tile's rows start no later and
    // end no later than the long one's
    const int klo = first_key(p.start_pos + ts0, p.window);
    kb = klo / BK;
    ke = (p.start_pos + tl1) / BK + 1;
    Tile t;
    t.kvh = kvh;
    t.split = 0;
    t.t0 = grp == 0 ? tl0 : ts0;
    t.t_last = grp == 0 ? tl1 : ts1;
    t.kt_begin = kb;
    t.kt_end = ke;
    t.klo = klo;
    t.kend = p.start_pos + tl1 + 1;
    return t;
}

// Per-lane row and per-wave token range.
struct Rows {
    int t, h, pos, lo;
    bool ok;                       // this lane's row exists
    bool wave_any;                 // the wave has at least one row
    bool wave_ragged;              // the wave has lanes without a row
    int w_pos_min, w_pos_max, w_lo_min, w_lo_max;
};

template <int RPW = kRowsPerWave>
__device__ inline Rows rows_of(const Params &p, const Tile &w, int wave, int lrow) {
    Rows r;
    const int n = wave * RPW + lrow;
    const int tl = n / p.G;
    r.t = w.t0 + tl;
    r.h = w.kvh * p.G + n % p.G;
    r.ok = tl < p.TQ && r.t <= w.t_last;
    r.pos = r.ok ? p.start_pos + r.t : -1;
    r.lo = r.ok ? first_key(r.pos, p.window) : 0;
    const int tf = w.t0 + (wave * RPW) / p.G;
    const int tl_last = min(w.t0 + (wave * RPW + RPW - 1) / p.G,
                            min(w.t0 + p.TQ - 1, w.t_last));
    r.wave_any = (wave * RPW) / p.G < p.TQ && tf <= w.t_last;
    r.wave_ragged = (wave * RPW + RPW - 1) / p.G >= p.TQ ||
                    w.t0 + (wave * RPW + RPW - 1) / p.G > w.t_last;
    r.w_pos_min = p.start_pos + tf;
    r.w_pos_max = p.start_pos + tl_last;
    r.w_lo_min = first_key(r.w_pos_min, p.window);
    r.w_lo_max = first_key(r.w_pos_max, p.window);
    return r;
}

// ---- epilogue shared by both kernels ----------------------------------------

// Value of lane l combined with lane l ^ 32 (the other half of the wave).
__device__ inline float max_halves(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ inline float sum_halves(float x) { return x + __shfl_xor(x, 32); }

template <int D>
__device__ inline void write_rows(const Params &p, const Tile &w, const Rows &r, int g,
                                  const f32x16 (&o)[D / 32], float mc, float lsum) {
    const float ltot = sum_halves(lsum);
    if (!r.ok) return;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (p.S == 1) {
        const int64_t e = (int64_t)r.t * p.out_row_stride + (int64_t)r.h * D + 4 * g;
        with_out_dtype(p.out_dtype, [&](auto ODT_) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 val = {o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv,
                                 o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv};
                    store_out4<decltype(ODT_)::value>(p.out, e + 32 * db + 8 * r4, val);
                }
        });
    } else {
        const int64_t row = (int64_t)w.split * p.T * p.H + (int64_t)r.t * p.H + r.h;
        float *dst = p.ws_o + row * D + 4 * g;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 val = {o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv,
                             o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv};
                *(f32x4 *)(dst + 32 * db + 8 * r4) = val;
            }
        if (g == 0) p.ws_ml[row] = make_float2(mc, ltot);
    }
}

// Online-softmax step for one tile: s holds raw scores (masked ones -inf).
// Returns alpha (the rescale of the previous accumulators) and updates m.
template <int NB>
__device__ inline float softmax_max(const f32x16 (&s)[NB], float &m, float c, float &mc) {
    float mt = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[b][i]);
    mt = max_halves(mt);
    const float mnew = fmaxf(m, mt);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f((m - muse) * c);
    m = mnew;
    mc = muse * c;
    return alpha;
}

// ---- bf16 / fp16 kernel -------------------------------------------------------
//
// K and V tiles go from HBM straight into LDS (buffer loads with the LDS
// destination, no register staging), double-buffered so that the loads of
// tile i+1 run under the math of tile i, with one barrier per tile.  The
// buffer descriptor of each kv head is limited to its L rows, so rows past
// L read as zero and are never fetched.  Both tiles are stored row-major
// ([key][d], 16-byte chunks) with an XOR swizzle of the chunk index instead
// of padding:
//   K: chunk c of row r sits at c ^ swz_k(r): the 16 rows one ds_read_b128
//      phase touches land in 16 different bank groups;
//   V: chunk c of row r sits at c ^ swz_v(r): the 4 rows x 4 chunks one
//      transposed read touches per half-wave land in 16 different groups.
// V^T operands come from ds_read_b64_tr_b16: inside each 16-lane group,
// output lane 4q+e gets element e of the rows addressed by lanes q, q+4,
// q+8, q+12, so lanes that address rows (key0 + 4*(l/32) + j/4) at column
// (d0 + 16*((l/16)%2) + 4*(j%4)), j = l%16, receive
// V[key0 + 4*(l/32) + r][d0 + l%32], r = 0..3: the A operand of V^T P^T.
// Operand reads run a few MFMAs ahead of their use (explicitly waited asm
// reads, see below), and the two S chains of a tile alternate so that each
// MFMA's accumulator was written two MFMAs earlier.  The row max of a tile
// combines the two lane halves with a lane swap instead of an LDS exchange.

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))
#define LDS_ADDR(a) ((__attribute__((address_space(3))) void *)(uintptr_t)(a))
#define LDS_I16X4(p) ((__attribute__((address_space(3))) i16x4 *)(p))

#if defined(__HIP_DEVICE_COMPILE__)   // buffer descriptors exist in the device pass only
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void *base, int bytes) {
    // raw buffer, stride 0, range `bytes` (gfx9 data-format word)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
#endif

[[maybe_unused]] __device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Largest K/V block per kv head the 16-bit kernels address (32-bit buffer
// offsets with room for a tile past its end), and an offset past any such
// range: loads there return zeros.
constexpr int kMaxHeadBytes = 0x7FE00000;
constexpr int kPastRange = 0x7FF00000;

// Ring cache (sliding-window layers): key j of a kv head sits in slot
// j % ring.  kend is the first key past the work-group's keys (at most L):
// rows at keys >= kend read as zero, like the rows past L of a linear cache.
// When the ring is a multiple of the tile and the tile ends before kend
// (ring_tile_linear), the tile's rows sit in consecutive slots from
// s0 = j0 % ring: the linear offsets with s0 rows added as the scalar offset.
// Otherwise ring_offsets: lin[i] is the offset lane load i of the tile would
// have in a linear cache, row * row_bytes + chunk; each row finds its slot
// s0 + row, wrapped once past the ring's end (rings of at least BK slots; the
// wrap test compares lin itself, since chunk < row_bytes) or reduced by
// division.  s0 is kept by the caller (ring_advance).
[[maybe_unused]] __device__ inline bool ring_tile_linear(const Params &p, int j0, int BK, int kend) {
    return p.ring % BK == 0 && j0 <= kend - BK;   // j0 + BK <= kend without forming it (may be 2^31)
}
template <int N>
__device__ inline void ring_offsets(const Params &p, int j0, int s0, int BK, int row_bytes, int kend,
                                    const int (&lin)[N], int (&off)[N]) {
    if (p.ring >= BK) {
        const int wrap_at = (p.ring - s0) * row_bytes, base = s0 * row_bytes;
        const int back = p.ring * row_bytes;
#pragma unroll
        for (int i = 0; i < N; ++i) off[i] = lin[i] + base - (lin[i] >= wrap_at ? back : 0);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int row = lin[i] / row_bytes;
            off[i] = ((s0 + row) % p.ring) * row_bytes + (lin[i] - row * row_bytes);
        }
    }
    if (j0 > kend - BK) {
        const int end = (kend - j0) * row_bytes;
#pragma unroll
        for (int i = 0; i < N; ++i) off[i] = lin[i] >= end ? kPastRange : off[i];
    }
}

// Slot of the first key of the next tile: a wavefront issues its tiles in
// order, so the slot moves by BK modulo the ring instead of a division per tile.
[[maybe_unused]] __device__ inline int ring_advance(int s, int BK, int ring) {
    const int n = s + BK;
    return n < ring ? n : ring >= BK ? n - ring : n % ring;
}

#if defined(__HIP_DEVICE_COMPILE__)
// Paged cache: the K/V descriptors of the tile whose first key is j0 (a page
// holds whole tiles), based at kv head kvh's rows of page `page` and covering
// the page's rows below kend (the first key past the work-group's keys, at
// most L), so rows at keys >= kend read as zero; an entry outside the pool
// reads as zeros.  soff = the tile's first row within the page.
__device__ inline void paged_rsrc(const Params &p, int kvh, int j0, int row_bytes, int page, int kend,
                                  __amdgpu_buffer_rsrc_t &rk, __amdgpu_buffer_rsrc_t &rv, int &soff) {
    const int r0 = j0 & ((1 << p.page_shift) - 1);
    const bool ok = page >= 0 && page < p.num_pages;
    const int rows = ok ? min(1 << p.page_shift, kend - (j0 - r0)) : 0;
    const int64_t base = ok ? ((((int64_t)page * p.KVH + kvh) << p.page_shift) * row_bytes) : 0;
    rk = head_rsrc((const uint8_t *)p.k + base, rows * row_bytes);
    rv = head_rsrc((const uint8_t *)p.v + base, rows * row_bytes);
    soff = r0 * row_bytes;
}

// The page of the tile whose first key is j (paged caches), -1 past L.
// (j in 64 bits: the tile after the last one may start at 2^31)
__device__ inline int page_of(const Params &p, int64_t j) {
    return j < p.L ? p.page_table[j >> p.page_shift] : -1;
}
#endif

// LDS operand reads issued as inline assembly.  The wait-count pass treats
// the builtin transposed read as one that may alias any LDS DMA still in
// flight and puts a vmcnt(0) in front of it, which would stall every P.V
// phase until the next tile's DMA (bound for the other buffer) has landed.
// The asm forms are invisible to that pass; their results are waited for
// with lds_wait, which ties the destination registers so that no user can be
// scheduled above the wait.
template <int OFF>
__device__ inline u32x2 ds_read_tr16(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
template <int OFF>
__device__ inline u32x4 ds_read_b128_asm(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
// Wait until at most N LDS operations of this wave are outstanding.  LDS
// operations return in order, so every read issued before the last N has
// landed (other lgkm traffic in between only makes the wait stricter).
template <int N>
__device__ inline void lds_wait(u32x2 &a, u32x2 &b) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ inline void lds_wait(u32x4 &a) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
// Maximum over the two 32-lane halves of a wave without an LDS round trip:
// the swap leaves x[l] and x[l ^ 32] in the two results of every lane.
[[maybe_unused]] __device__ inline float max_halves_swap(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Maximum over lanes l and l ^ 16 (the 16-lane rows of each half), likewise
// without LDS: the row swap leaves x[l] and x[l ^ 16] in the two results.
[[maybe_unused]] __device__ inline float max_quarters_swap(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max(a, b, c) as one v_max3_f32: written as fmaxf the compiler rebalances a
// row-max chain into two-operand maxima (0.75 instead of 0.5 instructions per
// score).  Scores are finite or -inf here.
[[maybe_unused]] __device__ inline float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
template <int I, int N, class F>
__device__ inline void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

template <int CPR>
__device__ inline int swz_k(int row) {
    if constexpr (CPR >= 16) return row & 15;
    else if constexpr (CPR == 8) return (row >> 1) & 7;
    else return (row >> 2) & 3;
}

template <int CPR>
__device__ inline int swz_v(int row) {
    if constexpr (CPR >= 16) return 4 * (row & 3);
    else if constexpr (CPR == 8) return 4 * ((row >> 1) & 1);
    else return 0;
}

struct Ones {
    __device__ static inline float dot(uint32_t p2, float acc, Bf16) {
        const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p2), one, acc, false);
    }
    __device__ static inline float dot(uint32_t p2, float acc, F16) {
        const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p2), one, acc, false);
    }
};

[[maybe_unused]] constexpr float kRescaleLog2 = 8.f;   // keep a stale row max while p <= 2^8

// ---- V in MFMA operand order ----------------------------------------------------
//
// The P.V product contracts over keys, so its A operand wants, per lane, eight
// keys of one head_dim column: a column of the row-major V cache.  LDS
// transposed reads deliver that at a third of the plain 128-bit read rate on
// gfx950, which made them the kernel's bottleneck.  This pass rewrites the V
// rows of the call's KV tiles once per call, in the order the operands are
// consumed: for each KV tile, each 16-byte chunk c = (block * steps + step) *
// 64 + lane holds the 8 values that lane feeds to one MFMA, so the attention
// kernels copy tiles into LDS verbatim and read each operand with one
// contiguous ds_read_b128.  Keys no row of the call reads (at or past L,
// below the first query's window) are written as zeros.  The copy is either
// per call (in the workspace, the call's tiles) or a mirror the caller keeps
// across the chunks of a sequence (key 0 up; each call rewrites only the
// tiles from the first key the mirror lacks, grid x = tiles rewritten).
//   M32 (32x32x16 MFMA): block = 32-wide d block, step = 16 keys; lane
//        (l%32, l/32), element e: key 16*step + 8*(e/4) + 4*(l/32) + e%4,
//        d = 32*block + l%32
//   M16 (16x16x32 MFMA): block = 16-wide d block, step = 32 keys; lane
//        (l%16, l/16), element e: key 32*step + 16*(e/4) + 4*(l/16) + e%4,
//        d = 16*block + l%16
template <int D, int BK, bool M16>
__global__ __launch_bounds__(256) void pack_v_operands(Params p, uint16_t *vop) {
    const uint16_t *v = (const uint16_t *)p.v;
    const int L = p.L, kt_lo = p.vop_kt_lo, ntiles = p.vop_tiles;
    const int jlo = first_key(p.start_pos, p.window);   // no row of the call reads keys below
    constexpr int PITCH = D + 2;               // LDS row pitch (elements): column reads spread banks
    constexpr int CHUNKS = BK * D / 8;
    __shared__ uint32_t t32[BK * PITCH / 2];
    const uint16_t *t16 = (const uint16_t *)t32;
    const int tile = p.vop_pack0 + blockIdx.x, kvh = blockIdx.y;
    const int j0 = (kt_lo + tile) * BK;
    for (int cidx = threadIdx.x; cidx < CHUNKS; cidx += 256) {
        const int key = cidx / (D / 8), c8 = cidx % (D / 8);
        const int j = j0 + key;
        const int64_t src = j >= jlo && j < L ? kv_row<D>(p, kvh, j) : -1;   // any cache layout
        const u32x4 val = src >= 0 ? *(const u32x4 *)(v + src + 8 * c8) : u32x4{0, 0, 0, 0};
        uint32_t *row = t32 + (key * PITCH + 8 * c8) / 2;
        row[0] = val[0];
        row[1] = val[1];
        row[2] = val[2];
        row[3] = val[3];
    }
    __syncthreads();
    uint16_t *dst = vop + ((int64_t)kvh * ntiles + tile) * (BK * D);
    for (int oc = threadIdx.x; oc < CHUNKS; oc += 256) {
        const int lane = oc % 64, op = oc / 64;
        int d, kbase, khalf;
        if (M16) {
            const int db = op / (BK / 32), kp = op % (BK / 32);
            d = 16 * db + (lane & 15);
            kbase = 32 * kp + 4 * (lane >> 4);
            khalf = 16;
        } else {
            const int db = op / (BK / 16), ks = op % (BK / 16);
            d = 32 * db + (lane & 31);
            kbase = 16 * ks + 4 * (lane >> 5);
            khalf = 8;
        }
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int k0 = kbase + khalf * (e / 4) + (e % 4);
            w[e / 2] = (uint32_t)t16[k0 * PITCH + d] | ((uint32_t)t16[(k0 + 1) * PITCH + d] << 16);
        }
        *(u32x4 *)(dst + 8 * oc) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

template <class Ty, int D, int BK, int NW, int WAVES_PER_SIMD, int LAYOUT>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD)))
void attn_fwd16(Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
    take_device_start(p);
    static_assert(D % 32 == 0 && BK % 32 == 0, "tile shape");
    constexpr int CPR = D / 8;                        // 16-byte chunks per row
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int TILE_CHUNKS = BK * CPR;
    constexpr int TILE_BYTES = TILE_CHUNKS * 16;
    constexpr int LOADS = TILE_CHUNKS / (NW * kWave);      // per wave, per matrix, per tile
    static_assert(LOADS >= 1 && LOADS * NW * kWave == TILE_CHUNKS, "staging split");
    constexpr int NB = BK / 32;                       // 32-key blocks per tile
    constexpr int NKB = D / 16 < 8 ? D / 16 : 8;      // distinct K read bases per lane
    constexpr int NVB = D / 32 < 4 ? D / 32 : 4;      // distinct V read bases per lane

    // [K buffer 0, K buffer 1][V buffer 0, V buffer 1]
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches, M0
    const int l32 = lane & 31, g = lane >> 5;
    int kb_all = 0, ke_all = 0;      // the work-group's KV tiles
    Tile w;
    if (NW == 8 && p.pair) {
        w = locate_pair<BK>(p, wave >> 2, kb_all, ke_all);
    } else {
        w = locate<BK>(p);
        kb_all = w.kt_begin;
        ke_all = w.kt_end;
    }
    const Rows r = rows_of(p, w, (NW == 8 && p.pair) ? (wave & 3) : wave, l32);
    // a linear cache's descriptors end at the work-group's last key (rows past
    // it read as zero); a ring's cover its slots (ring_offsets cuts them)
    const int kv_range = LAYOUT == kLinear ? w.kend * ROW_BYTES : p.kv_bytes;
    const __amdgpu_buffer_rsrc_t rk =
        head_rsrc((const uint16_t *)p.k + (int64_t)w.kvh * p.kv_head_stride, kv_range);
    const __amdgpu_buffer_rsrc_t rv =
        head_rsrc((const uint16_t *)p.v + (int64_t)w.kvh * p.kv_head_stride, kv_range);

    // DMA source offsets (bytes, relative to the tile's first row) of this lane
    int koff[LOADS], voff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int pos = (wave * LOADS + i) * kWave + lane;
        const int row = pos / CPR, cs = pos % CPR;
        koff[i] = row * D * 2 + ((cs ^ swz_k<CPR>(row)) * 16);
        voff[i] = row * D * 2 + ((cs ^ swz_v<CPR>(row)) * 16);
    }
    // LDS read offsets (bytes within a tile).  K: chunk 2ks+g of row l32 sits at
    // (2ks+g) ^ swz_k(l32); the swizzle only touches the low four chunk bits, so
    // step ks = 8u + v reads kbase[v] + 256u.  V: the transposed read of d-block
    // db at key 0 is vbase[db % 4] + 256 (db / 4), since swz_v only touches chunk
    // bits 2-3.  Everything else is an immediate offset.
    int kbase[NKB], vbase[NVB];
#pragma unroll
    for (int v = 0; v < NKB; ++v)
        kbase[v] = l32 * ROW_BYTES + (((2 * v + g) ^ swz_k<CPR>(l32)) * 16);
    {
        const int trow = 4 * g + (lane & 15) / 4;
        const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int db = 0; db < NVB; ++db) {
            const int d = 32 * db + tcol;
            vbase[db] = trow * ROW_BYTES + (((d >> 3) ^ swz_v<CPR>(trow)) * 16) + (d & 7) * 2;
        }
    }
    constexpr int PV_AHEAD = 4, S_AHEAD = 4;
    uint32_t vaddr[NVB], kaddr[NKB];
    {
        const uint32_t lds0 = (uint32_t)(uintptr_t)LDS_PTR(smem);
#pragma unroll
        for (int db = 0; db < NVB; ++db) vaddr[db] = lds0 + vbase[db];
#pragma unroll
        for (int v = 0; v < NKB; ++v) kaddr[v] = lds0 + kbase[v];
    }

    u32x4 qreg[D / 16];
    // Q rows, loaded after the first K/V tile's DMA has been issued so that
    // the two HBM round trips overlap
    auto load_q = [&]() {
        const uint16_t *qp = (const uint16_t *)p.q + (int64_t)(r.ok ? r.t : 0) * p.q_row_stride +
                             (int64_t)r.h * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qreg[ks] = r.ok ? *(const u32x4 *)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
        // Q * log2(e)/sqrt(D), rounded to the storage type: the products
        // then deliver scores in log2 units
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) qreg[ks][e] = Ty::scale2(qreg[ks][e], p.c);
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float mref = -INFINITY;          // reference row max, log2 units (raw score * c)
    float lsum = 0.f;                // this lane's share of the row sum
    // The score chains start from -mref (0 while mref is -inf), so each
    // product chain ends at s*c - mref, the exponent itself; zc holds that
    // start in every accumulator slot and changes only when mref moves.
    float zval = 0.f;
    f32x16 zc = f32x16{};
    float thr = -INFINITY;           // move mref when the tile max (minus mref) passes this

    int pg_next = -1;   // paged caches: page of the next tile this wave issues
    int ring_s = 0;     // ring caches: slot of the next tile's first key
    // Issue the DMA of KV tile kt into the K and V buffers at kdst / vdst.
    // FIRST (the work-group's first tile): rows below w.klo get an offset
    // past the descriptor's range, so they arrive as zeros.
    auto issue = [&](int kt, int kdst, int vdst, auto FIRST_) {
        constexpr bool FIRST = decltype(FIRST_)::value;
        // LDS destination (M0) of this wave's chunks: one scalar base, made
        // opaque at every issue so that the compiler derives the per-chunk
        // values here instead of keeping all sixteen live through the loop
        uint32_t mb = (uint32_t)(uintptr_t)LDS_PTR(smem) + wave * LOADS * 1024;
        asm volatile("" : "+s"(mb));
        // per-lane offsets with the tile's scalar base folded in, rows below
        // klo cut off (first tile only)
        auto cut = [&](const int (&in)[LOADS], int (&o)[LOADS], int base) {
            const int lim = (w.klo - kt * BK) * ROW_BYTES;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) o[i] = in[i] < lim ? kPastRange : in[i] + base;
        };
        if constexpr (LAYOUT == kLinear) {
            const int base = kt * BK * D * 2;
            if constexpr (FIRST) {
                int ko[LOADS], vo[LOADS];
                cut(koff, ko, base);
                cut(voff, vo, base);
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rk, LDS_ADDR(mb + kdst + i * 1024), 16, ko[i], 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, LDS_ADDR(mb + vdst + i * 1024), 16, vo[i], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rk, LDS_ADDR(mb + kdst + i * 1024), 16, koff[i], base, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, LDS_ADDR(mb + vdst + i * 1024), 16, voff[i], base, 0, 0);
                }
            }
        } else if constexpr (LAYOUT == kPaged) {
            __amdgpu_buffer_rsrc_t pk, pv;
            int soff;
            paged_rsrc(p, w.kvh, kt * BK, D * 2, pg_next, w.kend, pk, pv, soff);
            if constexpr (FIRST) {
                int ko[LOADS], vo[LOADS];
                cut(koff, ko, soff);
                cut(voff, vo, soff);
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        pk, LDS_ADDR(mb + kdst + i * 1024), 16, ko[i], 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        pv, LDS_ADDR(mb + vdst + i * 1024), 16, vo[i], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        pk, LDS_ADDR(mb + kdst + i * 1024), 16, koff[i], soff, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        pv, LDS_ADDR(mb + vdst + i * 1024), 16, voff[i], soff, 0, 0);
                }
            }
            pg_next = page_of(p, (int64_t)(kt + 1) * BK);     // one tile ahead of its use
        } else {
            const int s0 = ring_s, j0 = kt * BK;
            ring_s = ring_advance(ring_s, BK, p.ring);
            if (!FIRST && ring_tile_linear(p, j0, BK, w.kend)) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rk, LDS_ADDR(mb + kdst + i * 1024), 16, koff[i], s0 * D * 2, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, LDS_ADDR(mb + vdst + i * 1024), 16, voff[i], s0 * D * 2, 0, 0);
                }
            } else {
                int ko[LOADS], vo[LOADS];
                ring_offsets(p, j0, s0, BK, D * 2, w.kend, koff, ko);
                ring_offsets(p, j0, s0, BK, D * 2, w.kend, voff, vo);
                if constexpr (FIRST) {
                    const int lim = (w.klo - j0) * ROW_BYTES;
#pragma unroll
                    for (int i = 0; i < LOADS; ++i) {
                        ko[i] = koff[i] < lim ? kPastRange : ko[i];
                        vo[i] = voff[i] < lim ? kPastRange : vo[i];
                    }
                }
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rk, LDS_ADDR(mb + kdst + i * 1024), 16, ko[i], 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, LDS_ADDR(mb + vdst + i * 1024), 16, vo[i], 0, 0, 0);
                }
            }
        }
    };

    // one KV tile from the LDS buffers at byte offsets KO (K) and VO (V)
    auto tile = [&](auto KO_, auto VO_, int kt) {
        constexpr int KO = decltype(KO_)::value, VO = decltype(VO_)::value;
        const int j0 = kt * BK;
        if (!r.wave_any || j0 > r.w_pos_max || j0 + BK - 1 < r.w_lo_min) return;
        f32x16 s[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) s[b] = zc;
        {
            // S^T = K Q^T: the NB chains interleaved, operand reads S_AHEAD
            // products ahead of the matrix core
            constexpr int NS = NB * (D / 16);
            u32x4 ka[NS];
            auto kread = [&](auto I_) {
                constexpr int i = decltype(I_)::value, ks = i / NB, b = i % NB;
                ka[i] = ds_read_b128_asm<KO + 32 * b * ROW_BYTES + 256 * (ks / NKB)>(kaddr[ks % NKB]);
            };
            static_for<0, (S_AHEAD < NS ? S_AHEAD : NS)>(kread);
            static_for<0, NS>([&](auto I_) {
                constexpr int i = decltype(I_)::value, ks = i / NB, b = i % NB;
                if constexpr (i + S_AHEAD < NS) kread(std::integral_constant<int, i + S_AHEAD>{});
                constexpr int later = (NS - 1 - i) < S_AHEAD ? (NS - 1 - i) : S_AHEAD;
                lds_wait<later>(ka[i]);
                s[b] = Ty::mma(ka[i], qreg[ks], s[b]);
            });
        }
        // first V^T operands of this tile, in flight under the softmax
        constexpr int KSV = BK / 16, NPV = (D / 32) * KSV;
        u32x2 ta[NPV], tb[NPV];
        auto vread = [&](auto I_) {
            constexpr int i = decltype(I_)::value, db = i / KSV, ks = i % KSV;
            constexpr int off = VO + 16 * ks * ROW_BYTES + 256 * (db / NVB);
            ta[i] = ds_read_tr16<off>(vaddr[db % NVB]);
            tb[i] = ds_read_tr16<off + 8 * ROW_BYTES>(vaddr[db % NVB]);
        };
        static_for<0, (PV_AHEAD < NPV ? PV_AHEAD : NPV)>(vread);
        if (r.wave_ragged || j0 < r.w_lo_max || j0 + BK - 1 > r.w_pos_min) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j0 + 32 * b + (i / 4) * 8 + 4 * g + (i % 4);
                    if (key < r.lo || key > r.pos) s[b][i] = -INFINITY;
                }
        }
        // row max of the tile (raw scores), both lane halves; two independent
        // v_max3 chains so that no instruction waits on the one before it
        float mt0 = -INFINITY, mt1 = -INFINITY;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                mt0 = max3(mt0, s[b][i], s[b][i + 1]);
                mt1 = max3(mt1, s[b][i + 2], s[b][i + 3]);
            }
        const float mt = max_halves_swap(fmaxf(mt0, mt1));
        // move the reference max only when p could exceed 2^8 (exact either
        // way), or for the first keys a row sees
        if (__builtin_amdgcn_ballot_w64(mt > thr) != 0) {
            const float mnew = fmaxf(mref, mt - zval);
            if (mnew != -INFINITY) {
                const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
                const float shift = zval + mnew;
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[b][i] -= shift;
                mref = mnew;
                zval = -mnew;
                thr = kRescaleLog2;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
#pragma unroll
                for (int i = 0; i < 16; ++i) zc[i] = zval;
            }
        }
        u32x4 pb[BK / 16];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int i0 = 8 * half + 2 * jj;
                    const float p0 = __builtin_amdgcn_exp2f(s[b][i0]);
                    const float p1 = __builtin_amdgcn_exp2f(s[b][i0 + 1]);
                    const uint32_t pk = Ty::pack(p0, p1);
                    pb[2 * b + half][jj] = pk;
                    lsum = Ones::dot(pk, lsum, Ty{});
                }
        // O^T += V^T P^T: NPV products, their operand reads kept PV_AHEAD
        // products ahead of the matrix core
        static_for<0, NPV>([&](auto I_) {
            constexpr int i = decltype(I_)::value, db = i / KSV, ks = i % KSV;
            if constexpr (i + PV_AHEAD < NPV) vread(std::integral_constant<int, i + PV_AHEAD>{});
            constexpr int later = (NPV - 1 - i) < PV_AHEAD ? (NPV - 1 - i) : PV_AHEAD;
            lds_wait<2 * later>(ta[i], tb[i]);
            o[db] = Ty::mma(u32x4{ta[i][0], ta[i][1], tb[i][0], tb[i][1]}, pb[ks], o[db]);
        });
    };

    const int kb0 = kb_all, ke = ke_all;
    using B0K = std::integral_constant<int, 0>;
    using B1K = std::integral_constant<int, TILE_BYTES>;
    using B0V = std::integral_constant<int, 2 * TILE_BYTES>;
    using B1V = std::integral_constant<int, 3 * TILE_BYTES>;
    using First = std::true_type;
    using Next = std::false_type;
    if (kb0 < ke) {
        if constexpr (LAYOUT == kPaged) pg_next = page_of(p, kb0 * BK);
        if constexpr (LAYOUT == kRing) ring_s = kb0 * BK % p.ring;
        issue(kb0, B0K::value, B0V::value, First{});
        load_q();
        wait_vmem();
        __syncthreads();
        for (int kt = kb0; kt < ke; kt += 2) {
            // tile kt in buffer 0 while tile kt+1 streams into buffer 1
            if (kt + 1 < ke) issue(kt + 1, B1K::value, B1V::value, Next{});
            tile(B0K{}, B0V{}, kt);
            wait_vmem();
            __syncthreads();
            if (kt + 1 >= ke) break;
            // tile kt+1 in buffer 1 while tile kt+2 streams into buffer 0
            if (kt + 2 < ke) issue(kt + 2, B0K::value, B0V::value, Next{});
            tile(B1K{}, B1V{}, kt + 1);
            wait_vmem();
            __syncthreads();
        }
    }
    write_rows<D>(p, w, r, g, o, mref, lsum);
#endif
}

// ---- bf16 / fp16 kernel, 16 rows per wavefront (head_dim 256 and 512) ----------
//
// At head_dim 512 one wavefront cannot hold 32 rows of fp32 O (512 registers)
// next to its Q rows.  Here each of 8 wavefronts owns 16 rows and the
// products run on v_mfma_f32_16x16x32 (accumulator lane l, register i: row
// 4*(l/16) + i, column l%16):
//   S^T block (16 keys x 16 rows) = K Q^T, k = head_dim in steps of 32;
//   each lane holds 4 keys of one row per block, so the row max and sum
//   combine the four lane groups (l/16) with two exchanges;
//   O^T block (16 d x 16 rows) += V^T P^T, k = 32 keys: P comes from two S^T
//   blocks in the B-operand layout (slot (l/16, j): key 16*(j/4) + 4*(l/16) +
//   j%4).
// V^T operands (VPACK false, head_dim 256): two transposed LDS reads of the
// row-major V tile, which is swizzled for them: chunk c of row r sits at
// c ^ (2 * (r % 8)), so the 8 rows x 32 bytes a half-wave reads per
// transposed load fall in 16 different bank groups.  VPACK true (head_dim
// 512, where those reads bound the loop): the tiles come from the per-call
// copy in operand order (pack_v_operands) and each operand is one
// ds_read_b128; the copy costs a pass over the call's V rows, which only pays
// off when each row is reused by many query tiles.

constexpr int kWaves16 = 8;
constexpr int kThreads16 = kWaves16 * kWave;
constexpr int kRowsPerWave16 = 16;
static_assert(kWaves16 * kRowsPerWave16 == kRowsPerGroup, "same rows per work-group");

typedef float f32x4v __attribute__((ext_vector_type(4)));

struct Bf16m16 {
    __device__ static inline f32x4v mma(u32x4 a, u32x4 b, f32x4v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
struct F16m16 {
    __device__ static inline f32x4v mma(u32x4 a, u32x4 b, f32x4v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <class Ty> struct M16;
template <> struct M16<Bf16> { using T = Bf16m16; };
template <> struct M16<F16> { using T = F16m16; };

template <int CPR>
__device__ inline int swz_v16(int row) {
    static_assert(CPR >= 16, "head_dim >= 128");
    return 2 * (row & 7);
}

template <class Ty, int D, int BK, bool VPACK, int KSPLIT, int LAYOUT>
__global__ __launch_bounds__(kThreads16) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd16_r16(Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr bool SEED = D < 512;   // scores start from -mref (see below)
    take_device_start(p);
    static_assert(D >= 128 && D % 32 == 0 && BK % 32 == 0, "tile shape");
    static_assert(KSPLIT == 1 || (KSPLIT == 2 && !VPACK), "key halves read V in place");
    constexpr int NWH = kWaves16 / KSPLIT;            // wavefronts per key half
    using MM = typename M16<Ty>::T;
    constexpr int CPR = D / 8;
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int TILE_CHUNKS = BK * CPR;
    constexpr int TILE_BYTES = TILE_CHUNKS * 16;
    constexpr int LOADS = TILE_CHUNKS / (NWH * kWave);
    static_assert(LOADS * NWH * kWave == TILE_CHUNKS, "staging split");
    constexpr int NKS = D / 32;                       // k steps of S
    constexpr int NDB = D / 16;                       // 16-wide d blocks of O
    constexpr int NSB = BK / 16;                      // 16-key blocks of S per tile

    // per key half: [K buffer 0, K buffer 1, V buffer 0, V buffer 1]
    __shared__ __attribute__((aligned(1024))) uint8_t smem[KSPLIT * 4 * TILE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = KSPLIT == 1 ? 0 : wave / NWH;    // key half
    const int hw = KSPLIT == 1 ? wave : wave % NWH;   // wavefront within it
    uint8_t *const sm = KSPLIT == 1 ? smem : smem + half * 4 * TILE_BYTES;
    const int l16 = lane & 15, g4 = lane >> 4;
    const Tile w = locate<BK>(p);
    const Rows r = rows_of<kRowsPerWave16>(p, w, hw, l16);
    // a linear cache's descriptors end at the work-group's last key (rows past
    // it read as zero); a ring's cover its slots (ring_offsets cuts them); the
    // operand-order V copy holds zeros at keys no row of the call reads
    const int kv_range = LAYOUT == kLinear ? w.kend * ROW_BYTES : p.kv_bytes;
    const __amdgpu_buffer_rsrc_t rk =
        head_rsrc((const uint16_t *)p.k + (int64_t)w.kvh * p.kv_head_stride, kv_range);
    const __amdgpu_buffer_rsrc_t rv =
        VPACK ? head_rsrc(p.vop + (int64_t)w.kvh * p.vop_tiles * (BK * D), p.vop_tiles * TILE_BYTES)
              : head_rsrc((const uint16_t *)p.v + (int64_t)w.kvh * p.kv_head_stride, kv_range);

    int koff[LOADS], voff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int pos = (hw * LOADS + i) * kWave + lane;
        const int row = pos / CPR, cs = pos % CPR;
        koff[i] = row * D * 2 + ((cs ^ swz_k<CPR>(row)) * 16);
        voff[i] = VPACK ? pos * 16                    // operand-ordered V: verbatim copy
                        : row * D * 2 + ((cs ^ swz_v16<CPR>(row)) * 16);
    }
    // K: chunk 4ks + g4 of row 16b + l16 sits at (4ks + g4) ^ l16: the XOR only
    // touches chunk bits 0-3, so step ks = 4u + v reads kbase[v] + 256u.
    // V (VPACK): operand (db, kp) of this lane is chunk (db * BK/32 + kp) * 64 + lane.
    // V (transposed reads): d-block db at key 0 is read at rows 4*g4 + l16/4,
    // d = 16 db + 4 (lane%4); the XOR 2*(row%8) touches chunk bits 1-3, so
    // block db = 8u + v reads vaddr[v] + 256u.  vaddr holds the address in
    // the first V buffer; the buffer offset goes into the immediate.
    int kbase[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) kbase[v] = l16 * ROW_BYTES + (((4 * v + g4) ^ swz_k<CPR>(l16)) * 16);
    const int vlane = lane * 16;
    uint32_t kaddr[4];
    {
        const uint32_t lds0 = (uint32_t)(uintptr_t)LDS_PTR(sm);
#pragma unroll
        for (int v = 0; v < 4; ++v) kaddr[v] = lds0 + kbase[v];
    }
    constexpr int NVB16 = NDB < 8 ? NDB : 8;
    uint32_t vaddr[VPACK ? 1 : NVB16];
    if constexpr (VPACK) {
        vaddr[0] = (uint32_t)(uintptr_t)LDS_PTR(sm) + 2 * TILE_BYTES + vlane;
    } else {
        const uint32_t v0 = (uint32_t)(uintptr_t)LDS_PTR(sm) + 2 * TILE_BYTES;
        const int trow = 4 * g4 + l16 / 4;
#pragma unroll
        for (int v = 0; v < NVB16; ++v) {
            const int d = 16 * v + 4 * (lane & 3);
            vaddr[v] = v0 + trow * ROW_BYTES + (((d >> 3) ^ swz_v16<CPR>(trow)) * 16) + (d & 7) * 2;
        }
    }

    u32x4 qreg[NKS];
    // Q rows, loaded after the first K/V tile's DMA has been issued so that
    // the two HBM round trips overlap
    auto load_q = [&]() {
        const uint16_t *qp = (const uint16_t *)p.q + (int64_t)(r.ok ? r.t : 0) * p.q_row_stride +
                             (int64_t)r.h * D + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qreg[ks] = r.ok ? *(const u32x4 *)(qp + 32 * ks) : u32x4{0, 0, 0, 0};
        // Q * log2(e)/sqrt(D), rounded to the storage type: the products
        // then deliver scores in log2 units
        if constexpr (SEED) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) qreg[ks][e] = Ty::scale2(qreg[ks][e], p.c);
        }
    };

    f32x4v o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4v{0.f, 0.f, 0.f, 0.f};
    float mref = -INFINITY, lsum = 0.f;
    // SEED: the score chains start from -mref (0 while mref is -inf), so each
    // chain ends at the exponent s*c - mref; zc changes only when mref moves.
    // Otherwise (head_dim 512, where four more registers would spill) the
    // chains start from 0 and one FMA per score applies the scale and max.
    float zval = 0.f, thr = -INFINITY;
    f32x4v zc = f32x4v{0.f, 0.f, 0.f, 0.f};
    const float c = p.c;

    int pg_next = -1;   // paged caches: page of the next tile this wave issues
    int ring_s = 0;     // ring caches: slot of the next tile's first key
    // Issue the DMA of KV tile kt into the K and V buffers at kdst / vdst.
    // FIRST (a key half's first tile): rows below w.klo get an offset past the
    // descriptor's range, so they arrive as zeros (the operand-order V copy
    // already holds zeros there).
    auto issue = [&](int kt, int kdst, int vdst, auto FIRST_) {
        constexpr bool FIRST = decltype(FIRST_)::value;
        // per-lane offsets with the tile's scalar base folded in, rows below
        // klo cut off (first tile only)
        auto cut = [&](const int (&in)[LOADS], int (&o)[LOADS], int base) {
            const int lim = (w.klo - kt * BK) * ROW_BYTES;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) o[i] = in[i] < lim ? kPastRange : in[i] + base;
        };
        if constexpr (LAYOUT == kLinear) {
            const int base = kt * BK * D * 2;
            const int vbase_t = VPACK ? (kt - p.vop_kt_lo) * TILE_BYTES : base;
            int ko[LOADS], vo[LOADS];
            if constexpr (FIRST) {
                cut(koff, ko, base);
                if constexpr (!VPACK) cut(voff, vo, base);
            }
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rk, LDS_PTR(sm + kdst + (hw * LOADS + i) * 1024), 16, FIRST ? ko[i] : koff[i],
                    FIRST ? 0 : base, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, LDS_PTR(sm + vdst + (hw * LOADS + i) * 1024), 16,
                    FIRST && !VPACK ? vo[i] : voff[i], FIRST && !VPACK ? 0 : vbase_t, 0, 0);
            }
        } else if constexpr (LAYOUT == kPaged) {
            // the operand-ordered V copy is linear in the call's tiles
            __amdgpu_buffer_rsrc_t pk, pv;
            int soff;
            paged_rsrc(p, w.kvh, kt * BK, D * 2, pg_next, w.kend, pk, pv, soff);
            int ko[LOADS], vo[LOADS];
            if constexpr (FIRST) {
                cut(koff, ko, soff);
                if constexpr (!VPACK) cut(voff, vo, soff);
            }
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    pk, LDS_PTR(sm + kdst + (hw * LOADS + i) * 1024), 16, FIRST ? ko[i] : koff[i],
                    FIRST ? 0 : soff, 0, 0);
                if constexpr (VPACK)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, LDS_PTR(sm + vdst + (hw * LOADS + i) * 1024), 16, voff[i],
                        (kt - p.vop_kt_lo) * TILE_BYTES, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        pv, LDS_PTR(sm + vdst + (hw * LOADS + i) * 1024), 16, FIRST ? vo[i] : voff[i],
                        FIRST ? 0 : soff, 0, 0);
            }
            pg_next = page_of(p, (int64_t)(kt + 1) * BK);     // one tile ahead of its use
        } else {
            // the operand-ordered V copy is linear in the call's tiles; K (and
            // V read in place) come from the ring slots
            const int s0 = ring_s, j0 = kt * BK;
            ring_s = ring_advance(ring_s, BK, p.ring);
            const int vpack_base = (kt - p.vop_kt_lo) * TILE_BYTES;
            if (!FIRST && ring_tile_linear(p, j0, BK, w.kend)) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rk, LDS_PTR(sm + kdst + (hw * LOADS + i) * 1024), 16, koff[i], s0 * D * 2, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, LDS_PTR(sm + vdst + (hw * LOADS + i) * 1024), 16, voff[i],
                        VPACK ? vpack_base : s0 * D * 2, 0, 0);
                }
            } else {
                int ko[LOADS], vo[LOADS];
                ring_offsets(p, j0, s0, BK, D * 2, w.kend, koff, ko);
                if constexpr (!VPACK) ring_offsets(p, j0, s0, BK, D * 2, w.kend, voff, vo);
                if constexpr (FIRST) {
                    const int lim = (w.klo - j0) * ROW_BYTES;
#pragma unroll
                    for (int i = 0; i < LOADS; ++i) {
                        ko[i] = koff[i] < lim ? kPastRange : ko[i];
                        if constexpr (!VPACK) vo[i] = voff[i] < lim ? kPastRange : vo[i];
                    }
                }
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rk, LDS_PTR(sm + kdst + (hw * LOADS + i) * 1024), 16, ko[i], 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, LDS_PTR(sm + vdst + (hw * LOADS + i) * 1024), 16, VPACK ? voff[i] : vo[i],
                        VPACK ? vpack_base : 0, 0, 0);
                }
            }
        }
    };

    auto tile = [&](auto KO_, auto VO_, int kt) {
        constexpr int KO = decltype(KO_)::value, VO = decltype(VO_)::value;
        const int j0 = kt * BK;
        if (!r.wave_any || j0 > r.w_pos_max || j0 + BK - 1 < r.w_lo_min) return;
        // S^T = K Q^T: the NSB chains interleaved, operand reads S_AHEAD
        // products ahead (16x16x32 products are short, so reads run further
        // ahead than in the 32-row kernel)
        f32x4v s[NSB];
#pragma unroll
        for (int b = 0; b < NSB; ++b) s[b] = zc;
        {
            constexpr int NS = NSB * NKS, S_AHEAD = 6;
            u32x4 ka[NS];
            auto kread = [&](auto I_) {
                constexpr int i = decltype(I_)::value, ks = i / NSB, b = i % NSB;
                ka[i] = ds_read_b128_asm<KO + 16 * b * ROW_BYTES + 256 * (ks / 4)>(kaddr[ks % 4]);
            };
            static_for<0, (S_AHEAD < NS ? S_AHEAD : NS)>(kread);
            static_for<0, NS>([&](auto I_) {
                constexpr int i = decltype(I_)::value, ks = i / NSB, b = i % NSB;
                if constexpr (i + S_AHEAD < NS) kread(std::integral_constant<int, i + S_AHEAD>{});
                constexpr int later = (NS - 1 - i) < S_AHEAD ? (NS - 1 - i) : S_AHEAD;
                lds_wait<later>(ka[i]);
                s[b] = MM::mma(ka[i], qreg[ks], s[b]);
            });
        }
        if (r.wave_ragged || j0 < r.w_lo_max || j0 + BK - 1 > r.w_pos_min) {
#pragma unroll
            for (int b = 0; b < NSB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = j0 + 16 * b + 4 * g4 + i;
                    if (key < r.lo || key > r.pos) s[b][i] = -INFINITY;
                }
        }
        float mt0 = -INFINITY, mt1 = -INFINITY;
#pragma unroll
        for (int b = 0; b < NSB; ++b) {
            mt0 = max3(mt0, s[b][0], s[b][1]);
            mt1 = max3(mt1, s[b][2], s[b][3]);
        }
        const float mt = max_halves_swap(max_quarters_swap(fmaxf(mt0, mt1))) * (SEED ? 1.f : c);
        if (!SEED && __builtin_amdgcn_ballot_w64(mt > mref + kRescaleLog2) != 0) {
            const float mnew = fmaxf(mref, mt);
            const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
            mref = mnew;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        }
        if (SEED && __builtin_amdgcn_ballot_w64(mt > thr) != 0) {
            const float mnew = fmaxf(mref, mt - zval);
            if (mnew != -INFINITY) {
                const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
                const float shift = zval + mnew;
#pragma unroll
                for (int b = 0; b < NSB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[b][i] -= shift;
                mref = mnew;
                zval = -mnew;
                thr = kRescaleLog2;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db] *= alpha;
                zc = f32x4v{zval, zval, zval, zval};
            }
        }
        const float mc = SEED || mref == -INFINITY ? 0.f : mref;
        u32x4 pb[BK / 32];
#pragma unroll
        for (int kp = 0; kp < BK / 32; ++kp)
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const f32x4v &sb = s[2 * kp + half];
                    const float p0 = __builtin_amdgcn_exp2f(SEED ? sb[2 * jj] : fmaf(sb[2 * jj], c, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(SEED ? sb[2 * jj + 1] : fmaf(sb[2 * jj + 1], c, -mc));
                    const uint32_t pk = Ty::pack(p0, p1);
                    pb[kp][2 * half + jj] = pk;
                    lsum = Ones::dot(pk, lsum, Ty{});
                }
        if constexpr (VPACK) {
            // operand-ordered V: one ds_read_b128 per product, PV_AHEAD ahead;
            // vaddr[0] addresses the first V buffer, the rest is immediate
            constexpr int NPV = NDB * (BK / 32), PV_AHEAD = 6;
            u32x4 va[NPV];
            auto vread = [&](auto I_) {
                constexpr int i = decltype(I_)::value;
                va[i] = ds_read_b128_asm<VO - 2 * TILE_BYTES + i * 1024>(vaddr[0]);
            };
            static_for<0, (PV_AHEAD < NPV ? PV_AHEAD : NPV)>(vread);
            static_for<0, NPV>([&](auto I_) {
                constexpr int i = decltype(I_)::value, db = i / (BK / 32), kp = i % (BK / 32);
                if constexpr (i + PV_AHEAD < NPV) vread(std::integral_constant<int, i + PV_AHEAD>{});
                constexpr int later = (NPV - 1 - i) < PV_AHEAD ? (NPV - 1 - i) : PV_AHEAD;
                lds_wait<later>(va[i]);
                o[db] = MM::mma(va[i], pb[kp], o[db]);
            });
        } else {
            // transposed reads, kept PV_AHEAD products ahead of the matrix core
            constexpr int NPV = NDB * (BK / 32), PV_AHEAD = 7;   // 14 reads in flight
            u32x2 ta[NPV], tb[NPV];
            auto vread = [&](auto I_) {
                constexpr int i = decltype(I_)::value, db = i / (BK / 32), kp = i % (BK / 32);
                constexpr int off = VO - 2 * TILE_BYTES + 32 * kp * ROW_BYTES + 256 * (db / NVB16);
                ta[i] = ds_read_tr16<off>(vaddr[db % NVB16]);
                tb[i] = ds_read_tr16<off + 16 * ROW_BYTES>(vaddr[db % NVB16]);
            };
            static_for<0, (PV_AHEAD < NPV ? PV_AHEAD : NPV)>(vread);
            static_for<0, NPV>([&](auto I_) {
                constexpr int i = decltype(I_)::value, db = i / (BK / 32), kp = i % (BK / 32);
                if constexpr (i + PV_AHEAD < NPV) vread(std::integral_constant<int, i + PV_AHEAD>{});
                constexpr int later = (NPV - 1 - i) < PV_AHEAD ? (NPV - 1 - i) : PV_AHEAD;
                lds_wait<2 * later>(ta[i], tb[i]);
                o[db] = MM::mma(u32x4{ta[i][0], ta[i][1], tb[i][0], tb[i][1]}, pb[kp], o[db]);
            });
        }
    };

    using B0K = std::integral_constant<int, 0>;
    using B1K = std::integral_constant<int, TILE_BYTES>;
    using B0V = std::integral_constant<int, 2 * TILE_BYTES>;
    using B1V = std::integral_constant<int, 3 * TILE_BYTES>;
    const int kb0 = w.kt_begin, ke = w.kt_end;
    using First = std::true_type;
    using Next = std::false_type;
    if constexpr (KSPLIT == 1) {
        if (kb0 < ke) {
            if constexpr (LAYOUT == kPaged) pg_next = page_of(p, kb0 * BK);
            if constexpr (LAYOUT == kRing) ring_s = kb0 * BK % p.ring;
            issue(kb0, B0K::value, B0V::value, First{});
            load_q();
            wait_vmem();
            __syncthreads();
            for (int kt = kb0; kt < ke; kt += 2) {
                if (kt + 1 < ke) issue(kt + 1, B1K::value, B1V::value, Next{});
                tile(B0K{}, B0V{}, kt);
                wait_vmem();
                __syncthreads();
                if (kt + 1 >= ke) break;
                if (kt + 2 < ke) issue(kt + 2, B0K::value, B0V::value, Next{});
                tile(B1K{}, B1V{}, kt + 1);
                wait_vmem();
                __syncthreads();
            }
        }
    } else {
        // the first half takes the first ceil(n/2) of the work-group's n KV
        // tiles, the second half the rest; both step through the same number
        // of iterations so that they share every barrier
        const int niter = (ke - kb0 + 1) / 2;
        const int hb = half == 1 ? kb0 + niter : kb0;
        const int he = half == 0 ? kb0 + niter : ke;
        if (niter > 0) {
            if constexpr (LAYOUT == kPaged) pg_next = hb < he ? page_of(p, hb * BK) : -1;
            if constexpr (LAYOUT == kRing) ring_s = hb * BK % p.ring;
            if (hb < he) issue(hb, B0K::value, B0V::value, First{});
            load_q();
            wait_vmem();
            __syncthreads();
            for (int it = 0; it < niter; it += 2) {
                const int kt = hb + it;
                if (kt + 1 < he) issue(kt + 1, B1K::value, B1V::value, Next{});
                if (kt < he) tile(B0K{}, B0V{}, kt);
                wait_vmem();
                __syncthreads();
                if (it + 1 >= niter) break;
                if (kt + 2 < he) issue(kt + 2, B0K::value, B0V::value, Next{});
                if (kt + 1 < he) tile(B1K{}, B1V{}, kt + 1);
                wait_vmem();
                __syncthreads();
            }
        }
    }

    if constexpr (KSPLIT == 2) {
        // the second half hands (O, m, l) of its rows to the wavefront of the
        // first half that holds the same rows (same hw and lane), as 16-byte
        // pieces (lane-consecutive); the buffers are free after the loop's
        // last barrier
        constexpr int NX = NDB + 1;
        static_assert(NWH * NX * kWave * 16 <= KSPLIT * 4 * TILE_BYTES, "exchange fits in LDS");
        f32x4 *xch = (f32x4 *)smem + hw * NX * kWave + lane;
        if (half == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) xch[db * kWave] = f32x4{o[db][0], o[db][1], o[db][2], o[db][3]};
            xch[NDB * kWave] = f32x4{mref, lsum, 0.f, 0.f};
        }
        __syncthreads();
        if (half == 0) {
            const f32x4 ml = xch[NDB * kWave];
            const float ms = fmaxf(mref, ml[0]);
            const float a0 = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref - ms);
            const float a1 = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - ms);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const f32x4 x = xch[db * kWave];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[db][i] = o[db][i] * a0 + x[i] * a1;
            }
            lsum = lsum * a0 + ml[1] * a1;
            mref = ms;
        }
    }

    // the row's sum is spread over the four lane groups
    float ltot = lsum + __shfl_xor(lsum, 16);
    ltot = ltot + __shfl_xor(ltot, 32);
    if (r.ok && (KSPLIT == 1 || half == 0)) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        if (p.S == 1) {
            const int64_t e = (int64_t)r.t * p.out_row_stride + (int64_t)r.h * D + 4 * g4;
            with_out_dtype(p.out_dtype, [&](auto ODT_) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    store_out4<decltype(ODT_)::value>(
                        p.out, e + 16 * db,
                        f32x4{o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv});
            });
        } else {
            const int64_t row = (int64_t)w.split * p.T * p.H + (int64_t)r.t * p.H + r.h;
            float *dst = p.ws_o + row * D + 4 * g4;
            if (g4 == 0) p.ws_ml[row] = make_float2(mref, ltot);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                *(f32x4 *)(dst + 16 * db) = f32x4{o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv};
        }
    }
#endif
}

// ---- fp32 kernel ---------------------------------------------------------------

__device__ inline f32x16 mma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, int BK>
__global__ __launch_bounds__(kThreads) void attn_fwd32(Params p) {
    static_assert(D % 32 == 0 && BK % 32 == 0, "tile shape");
    take_device_start(p);
    constexpr int KROW = D + 4;           // floats; 16 B of padding
    constexpr int VROW = BK + 4;
    constexpr int KVEC = BK * D / 4;
    constexpr int KPT = KVEC / kThreads;
    constexpr int VTASK = (BK / 4) * (D / 4);  // (key quad, 4-wide d chunk) tasks
    constexpr int VPT = (VTASK + kThreads - 1) / kThreads;
    constexpr int HALF = D / 2;           // k slot (l/32) = 0 takes d < D/2, 1 the rest
    static_assert(KPT * kThreads == KVEC, "staging split");
    static_assert(VTASK % kThreads == 0 || VTASK < kThreads, "staging split");

    __shared__ __attribute__((aligned(16))) float Ks[BK * KROW];
    __shared__ __attribute__((aligned(16))) float Vt[D * VROW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches, M0
    const int l32 = lane & 31, g = lane >> 5;
    const Tile w = locate<BK>(p);
    const Rows r = rows_of(p, w, wave, l32);

    float qreg[HALF];
    {
        const float *qp = (const float *)p.q + (int64_t)(r.ok ? r.t : 0) * p.q_row_stride +
                          (int64_t)r.h * D + HALF * g;
#pragma unroll
        for (int i = 0; i < HALF / 4; ++i) {
            const f32x4 v = r.ok ? *(const f32x4 *)(qp + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
            qreg[4 * i] = v[0];
            qreg[4 * i + 1] = v[1];
            qreg[4 * i + 2] = v[2];
            qreg[4 * i + 3] = v[3];
        }
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m = -INFINITY, lsum = 0.f;

    f32x4 kbuf[KPT];
    f32x4 vbuf[VPT][4];
    auto gload = [&](int kt) {
        const int j0 = kt * BK;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * kThreads;
            const int key = idx / (D / 4), c4 = idx % (D / 4);
            // keys the work-group's rows read, any cache layout; the rest load as zeros
            const int j = j0 + key;
            const int64_t row = j >= w.klo && j < w.kend ? kv_row<D>(p, w.kvh, j) : -1;
            kbuf[i] = row >= 0 ? *(const f32x4 *)((const float *)p.k + row + 4 * c4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + i * kThreads;
            if (VTASK < kThreads && idx >= VTASK) break;
            const int c4 = idx % (D / 4), kq = idx / (D / 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + 4 * kq + u;
                const int64_t row = j >= w.klo && j < w.kend ? kv_row<D>(p, w.kvh, j) : -1;
                vbuf[i][u] = row >= 0 ? *(const f32x4 *)((const float *)p.v + row + 4 * c4)
                                      : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * kThreads;
            const int key = idx / (D / 4), c4 = idx % (D / 4);
            *(f32x4 *)&Ks[key * KROW + 4 * c4] = kbuf[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + i * kThreads;
            if (VTASK < kThreads && idx >= VTASK) break;
            const int c4 = idx % (D / 4), kq = idx / (D / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f32x4 col = {vbuf[i][0][e], vbuf[i][1][e], vbuf[i][2][e], vbuf[i][3][e]};
                *(f32x4 *)&Vt[(4 * c4 + e) * VROW + 4 * kq] = col;
            }
        }
    };

    if (w.kt_begin < w.kt_end) {
        gload(w.kt_begin);
        for (int kt = w.kt_begin; kt < w.kt_end; ++kt) {
            __syncthreads();
            lstore();
            __syncthreads();
            if (kt + 1 < w.kt_end) gload(kt + 1);
            const int j0 = kt * BK;
            if (!r.wave_any || j0 > r.w_pos_max || j0 + BK - 1 < r.w_lo_min) continue;

            f32x16 s[BK / 32];
#pragma unroll
            for (int b = 0; b < BK / 32; ++b) {
                s[b] = f32x16{};
                const float *kp = &Ks[(32 * b + l32) * KROW + HALF * g];
#pragma unroll
                for (int st = 0; st < HALF; st += 4) {
                    const f32x4 a4 = *(const f32x4 *)(kp + st);
                    s[b] = mma_f32(a4[0], qreg[st], s[b]);
                    s[b] = mma_f32(a4[1], qreg[st + 1], s[b]);
                    s[b] = mma_f32(a4[2], qreg[st + 2], s[b]);
                    s[b] = mma_f32(a4[3], qreg[st + 3], s[b]);
                }
            }
            if (r.wave_ragged || j0 < r.w_lo_max || j0 + BK - 1 > r.w_pos_min) {
#pragma unroll
                for (int b = 0; b < BK / 32; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = j0 + 32 * b + (i / 4) * 8 + 4 * g + (i % 4);
                        if (key < r.lo || key > r.pos) s[b][i] = -INFINITY;
                    }
            }
            float mc;
            const float alpha = softmax_max<BK / 32>(s, m, p.c, mc);
            float ps = 0.f;
#pragma unroll
            for (int b = 0; b < BK / 32; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[b][i] = __builtin_amdgcn_exp2f(fmaf(s[b][i], p.c, -mc));
                    ps += s[b][i];
                }
            lsum = lsum * alpha + ps;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const float *vp = &Vt[(32 * db + l32) * VROW + 4 * g];
#pragma unroll
                for (int b = 0; b < BK / 32; ++b)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const f32x4 a4 = *(const f32x4 *)(vp + 32 * b + 8 * r4);
                        o[db] = mma_f32(a4[0], s[b][4 * r4], o[db]);
                        o[db] = mma_f32(a4[1], s[b][4 * r4 + 1], o[db]);
                        o[db] = mma_f32(a4[2], s[b][4 * r4 + 2], o[db]);
                        o[db] = mma_f32(a4[3], s[b][4 * r4 + 3], o[db]);
                    }
            }
        }
    }
    write_rows<D>(p, w, r, g, o, m * p.c, lsum);
}

// ---- split merge ------------------------------------------------------------------

// out(t, h, :) = sum_s w_s O_s / sum_s w_s with w_s = l_s * 2^(m_s - m*) (m in log2 units),
// m* the largest m_s among splits that saw a valid key (l_s > 0).
template <int D>
__global__ __launch_bounds__(256) void merge_splits(const float *ws_o, const float2 *ws_ml,
                                                    void *out, int out_dtype, int64_t out_row_stride,
                                                    int T, int H, int S, float c) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)T * H;
    const int64_t row = idx / (D / 4);
    const int d4 = (int)(idx % (D / 4));
    if (row >= rows) return;
    float mstar = -INFINITY;
    for (int s = 0; s < S; ++s) {
        const float2 ml = ws_ml[s * rows + row];
        if (ml.y > 0.f) mstar = fmaxf(mstar, ml.x);
    }
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
        const float2 ml = ws_ml[s * rows + row];
        if (ml.y > 0.f) {
            const float wgt = ml.y * __builtin_amdgcn_exp2f(ml.x - mstar);
            wsum += wgt;
            acc += wgt * *(const f32x4 *)(ws_o + (s * rows + row) * D + 4 * d4);
        }
    }
    const int t = (int)(row / H), h = (int)(row % H);
    const int64_t e = (int64_t)t * out_row_stride + (int64_t)h * D + 4 * d4;
    with_out_dtype(out_dtype, [&](auto ODT_) {
        store_out4<decltype(ODT_)::value>(out, e, acc * (1.f / wsum));
    });
}

// The same merge for many splits (short chunks over long caches): one
// work-group per (token, head) row, so that the splits are read in parallel
// rather than one after another by each thread.  Threads s < S weigh split s
// (after a work-group maximum of the m_s); then thread (g, d4) sums the
// splits s = g mod NG of column block d4 and the NG partial sums are added in
// LDS.
template <int D>
__global__ __launch_bounds__(512) void merge_splits_wide(const float *ws_o, const float2 *ws_ml,
                                                         void *out, int out_dtype,
                                                         int64_t out_row_stride, int T, int H, int S) {
    constexpr int C4 = D / 4, NG = 512 / C4;
    __shared__ float wts[512];
    __shared__ float red[512 / kWave];
    __shared__ f32x4 part[512];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rows = (int64_t)T * H, row = blockIdx.x;
    float2 ml = {-INFINITY, 0.f};
    if (tid < S) ml = ws_ml[tid * rows + row];
    // m* over the splits that saw a valid key
    float m = ml.y > 0.f ? ml.x : -INFINITY;
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    float mstar = red[0];
    for (int i = 1; i < 512 / kWave; ++i) mstar = fmaxf(mstar, red[i]);
    const float wgt = ml.y > 0.f ? ml.y * __builtin_amdgcn_exp2f(ml.x - mstar) : 0.f;
    wts[tid] = wgt;
    __syncthreads();
    float wsum = 0.f;
    for (int i = 0; i < S; ++i) wsum += wts[i];
    const int g = tid / C4, d4 = tid % C4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // eight splits' loads in flight per step (a split without a valid key for
    // this row has weight 0 and its partial row is never added)
    constexpr int U = 8;
    for (int s0 = g; s0 < S; s0 += U * NG) {
        f32x4 vals[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = s0 + u * NG;
            vals[u] = sp < S ? *(const f32x4 *)(ws_o + (sp * rows + row) * D + 4 * d4)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = s0 + u * NG;
            const float w = sp < S ? wts[sp] : 0.f;
            if (w > 0.f) acc += w * vals[u];
        }
    }
    part[tid] = acc;
    __syncthreads();
    if (g == 0) {
        for (int i = 1; i < NG; ++i) acc += part[i * C4 + d4];
        const int t = (int)(row / H), h = (int)(row % H);
        const int64_t e = (int64_t)t * out_row_stride + (int64_t)h * D + 4 * d4;
        with_out_dtype(out_dtype, [&](auto ODT_) {
            store_out4<decltype(ODT_)::value>(out, e, acc * (1.f / wsum));
        });
    }
}

// ---- KV cache write (companion kernel) -------------------------------------------------
//
// The step before the attention: each token of the chunk stores its K and V
// rows in the cache (the gnosis page, "What already shipped", Phase A; the
// TensorSharp page, section 4, requirement R4: global layers at row
// start_pos + i, sliding-window layers at slot (start_pos + i) % ring).
// Element e of the flat (token, kv head, 16-byte chunk) space of K, then of V,
// is one thread's 16-byte move; consecutive threads read consecutive bytes of
// a token's K (or V) block and write consecutive bytes of one cache row.  In a
// ring, a token that a later token of the same chunk overwrites is not written
// (only the last `ring` tokens are), which leaves what in-order writes leave.
__global__ __launch_bounds__(256) void kv_write(const uint8_t *k_src, const uint8_t *v_src,
                                                int64_t src_row_bytes, uint8_t *k_cache,
                                                uint8_t *v_cache, int64_t head_bytes, int row_bytes,
                                                int KVH, int t_first, int T, int start_pos, int ring) {
    const int cpr = row_bytes / 16;                       // chunks per cache row
    const int per_token = KVH * cpr;
    const int n = (T - t_first) * per_token;              // chunks of K (and of V)
    const int stride = (int)(gridDim.x * blockDim.x);
    for (int idx = (int)(blockIdx.x * blockDim.x + threadIdx.x); idx < 2 * n; idx += stride) {
        const bool is_v = idx >= n;
        const int e = is_v ? idx - n : idx;
        const int i = t_first + e / per_token;
        const int c = e - (i - t_first) * per_token;      // chunk within the token's block
        const int kh = c / cpr, cc = c - kh * cpr;
        const int64_t pos = (int64_t)start_pos + i;
        const int64_t slot = ring ? pos % ring : pos;
        const u32x4 val = *(const u32x4 *)((is_v ? v_src : k_src) + i * src_row_bytes + (int64_t)c * 16);
        *(u32x4 *)((is_v ? v_cache : k_cache) + kh * head_bytes + slot * row_bytes + (int64_t)cc * 16) = val;
    }
}

// ---- host side -----------------------------------------------------------------------

using KernelFn = void (*)(Params);
using PackFn = void (*)(Params, uint16_t *);

struct Variant {
    int dtype, D, BK;
    int groups_per_cu;         // resident work-groups per CU the kernel is sized for
    int threads;               // work-group size (4 or 8 wavefronts)
    int rows;                  // (token, head) rows per work-group
    int ksplit;                // 2: the tile's keys are split between two wavefront halves;
                               // 0: variant without the V operand-order copy, for few query tiles;
                               // 3: two query tiles per work-group sharing their KV tiles
    KernelFn fn;               // linear caches
    KernelFn fn_ring;          // ring caches (key j in slot j % ring)
    KernelFn fn_paged;         // paged caches (key j in page page_table[j / page_size])
    PackFn pack;               // V operand-order pass (16-bit inputs), else null
};

const Variant kVariants[] = {
    {PA_DTYPE_BF16, 32, 64, 2, kThreads, kRowsPerGroup, 1, attn_fwd16<Bf16, 32, 64, 4, 2, kLinear>, attn_fwd16<Bf16, 32, 64, 4, 2, kRing>, attn_fwd16<Bf16, 32, 64, 4, 2, kPaged>, nullptr},
    {PA_DTYPE_BF16, 64, 64, 2, kThreads, kRowsPerGroup, 1, attn_fwd16<Bf16, 64, 64, 4, 2, kLinear>, attn_fwd16<Bf16, 64, 64, 4, 2, kRing>, attn_fwd16<Bf16, 64, 64, 4, 2, kPaged>, nullptr},
    {PA_DTYPE_BF16, 128, 64, 2, kThreads, kRowsPerGroup, 1, attn_fwd16<Bf16, 128, 64, 4, 2, kLinear>, attn_fwd16<Bf16, 128, 64, 4, 2, kRing>, attn_fwd16<Bf16, 128, 64, 4, 2, kPaged>, nullptr},
    {PA_DTYPE_BF16, 128, 64, 1, 2 * kThreads, kRowsPerGroup, 3, attn_fwd16<Bf16, 128, 64, 8, 2, kLinear>, attn_fwd16<Bf16, 128, 64, 8, 2, kRing>, attn_fwd16<Bf16, 128, 64, 8, 2, kPaged>, nullptr},
    {PA_DTYPE_BF16, 256, 64, 1, kThreads16, kRowsPerGroup, 1, attn_fwd16_r16<Bf16, 256, 64, false, 1, kLinear>, attn_fwd16_r16<Bf16, 256, 64, false, 1, kRing>, attn_fwd16_r16<Bf16, 256, 64, false, 1, kPaged>, nullptr},
    {PA_DTYPE_BF16, 256, 32, 1, kThreads16, kRowsPerGroup / 2, 2, attn_fwd16_r16<Bf16, 256, 32, false, 2, kLinear>, attn_fwd16_r16<Bf16, 256, 32, false, 2, kRing>, attn_fwd16_r16<Bf16, 256, 32, false, 2, kPaged>, nullptr},
    {PA_DTYPE_BF16, 512, 32, 1, kThreads16, kRowsPerGroup, 1, attn_fwd16_r16<Bf16, 512, 32, true, 1, kLinear>, attn_fwd16_r16<Bf16, 512, 32, true, 1, kRing>, attn_fwd16_r16<Bf16, 512, 32, true, 1, kPaged>, pack_v_operands<512, 32, true>},
    {PA_DTYPE_BF16, 512, 32, 1, kThreads16, kRowsPerGroup, 0, attn_fwd16_r16<Bf16, 512, 32, false, 1, kLinear>, attn_fwd16_r16<Bf16, 512, 32, false, 1, kRing>, attn_fwd16_r16<Bf16, 512, 32, false, 1, kPaged>, nullptr},
    {PA_DTYPE_F16, 32, 64, 2, kThreads, kRowsPerGroup, 1, attn_fwd16<F16, 32, 64, 4, 2, kLinear>, attn_fwd16<F16, 32, 64, 4, 2, kRing>, attn_fwd16<F16, 32, 64, 4, 2, kPaged>, nullptr},
    {PA_DTYPE_F16, 64, 64, 2, kThreads, kRowsPerGroup, 1, attn_fwd16<F16, 64, 64, 4, 2, kLinear>, attn_fwd16<F16, 64, 64, 4, 2, kRing>, attn_fwd16<F16, 64, 64, 4, 2, kPaged>, nullptr},
    {PA_DTYPE_F16, 128, 64, 2, kThreads, kRowsPerGroup, 1, attn_fwd16<F16, 128, 64, 4, 2, kLinear>, attn_fwd16<F16, 128, 64, 4, 2, kRing>, attn_fwd16<F16, 128, 64, 4, 2, kPaged>, nullptr},
    {PA_DTYPE_F16, 128, 64, 1, 2 * kThreads, kRowsPerGroup, 3, attn_fwd16<F16, 128, 64, 8, 2, kLinear>, attn_fwd16<F16, 128, 64, 8, 2, kRing>, attn_fwd16<F16, 128, 64, 8, 2, kPaged>, nullptr},
    {PA_DTYPE_F16, 256, 64, 1, kThreads16, kRowsPerGroup, 1, attn_fwd16_r16<F16, 256, 64, false, 1, kLinear>, attn_fwd16_r16<F16, 256, 64, false, 1, kRing>, attn_fwd16_r16<F16, 256, 64, false, 1, kPaged>, nullptr},
    {PA_DTYPE_F16, 256, 32, 1, kThreads16, kRowsPerGroup / 2, 2, attn_fwd16_r16<F16, 256, 32, false, 2, kLinear>, attn_fwd16_r16<F16, 256, 32, false, 2, kRing>, attn_fwd16_r16<F16, 256, 32, false, 2, kPaged>, nullptr},
    {PA_DTYPE_F16, 512, 32, 1, kThreads16, kRowsPerGroup, 1, attn_fwd16_r16<F16, 512, 32, true, 1, kLinear>, attn_fwd16_r16<F16, 512, 32, true, 1, kRing>, attn_fwd16_r16<F16, 512, 32, true, 1, kPaged>, pack_v_operands<512, 32, true>},
    {PA_DTYPE_F16, 512, 32, 1, kThreads16, kRowsPerGroup, 0, attn_fwd16_r16<F16, 512, 32, false, 1, kLinear>, attn_fwd16_r16<F16, 512, 32, false, 1, kRing>, attn_fwd16_r16<F16, 512, 32, false, 1, kPaged>, nullptr},
    {PA_DTYPE_F32, 32, 32, 2, kThreads, kRowsPerGroup, 1, attn_fwd32<32, 32>, attn_fwd32<32, 32>, attn_fwd32<32, 32>, nullptr},
    {PA_DTYPE_F32, 64, 32, 2, kThreads, kRowsPerGroup, 1, attn_fwd32<64, 32>, attn_fwd32<64, 32>, attn_fwd32<64, 32>, nullptr},
    {PA_DTYPE_F32, 128, 32, 2, kThreads, kRowsPerGroup, 1, attn_fwd32<128, 32>, attn_fwd32<128, 32>, attn_fwd32<128, 32>, nullptr},
    {PA_DTYPE_F32, 256, 32, 1, kThreads, kRowsPerGroup, 1, attn_fwd32<256, 32>, attn_fwd32<256, 32>, attn_fwd32<256, 32>, nullptr},
};

using MergeFn = void (*)(const float *, const float2 *, void *, int, int64_t, int, int, int, float);
using WideMergeFn = void (*)(const float *, const float2 *, void *, int, int64_t, int, int, int);

// splits above which the merge reads them in parallel (merge_splits_wide)
constexpr int kWideMergeSplits = 8;

WideMergeFn wide_merge_for(int D) {
    switch (D) {
        case 32: return merge_splits_wide<32>;
        case 64: return merge_splits_wide<64>;
        case 128: return merge_splits_wide<128>;
        case 256: return merge_splits_wide<256>;
        case 512: return merge_splits_wide<512>;
    }
    return nullptr;
}

MergeFn merge_for(int D) {
    switch (D) {
        case 32: return merge_splits<32>;
        case 64: return merge_splits<64>;
        case 128: return merge_splits<128>;
        case 256: return merge_splits<256>;
        case 512: return merge_splits<512>;
    }
    return nullptr;
}

const Variant *find_variant(int dtype, int D) {
    for (const Variant &v : kVariants)
        if (v.dtype == dtype && v.D == D && v.ksplit == 1) return &v;
    return nullptr;
}

// The variant whose work-groups split each tile's keys between two halves of
// their wavefronts (ksplit 2), or the one that reads V in place instead of an
// operand-order copy (ksplit 0), if this dtype and head_dim have one.
const Variant *find_ksplit_variant(int dtype, int D, int ksplit = 2) {
    for (const Variant &v : kVariants)
        if (v.dtype == dtype && v.D == D && v.ksplit == ksplit) return &v;
    return nullptr;
}

int elem_bytes(int dtype) { return dtype == PA_DTYPE_F32 ? 4 : 2; }

struct Plan {
    const Variant *var;
    int G, TQ, nq, S, items;
    int64_t tiles;               // KV tiles visited by all work-groups
    int vop_kt_lo, vop_tiles;    // KV tiles held in operand order (16-bit inputs)
    size_t vop_bytes;            // their bytes, at the start of the workspace (0 with a mirror)
    void *vmirror = nullptr;     // the caller's operand-order copy of V (else the workspace)
    int pack0 = 0, npack = 0;    // tiles (from vop_kt_lo) the operand-order pass rewrites
    size_t ws_bytes, ws_o_offset, ws_ml_offset;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kMaxSplits = 256;
constexpr int kMinQueryTilesForPack = 8;

int first_key_host(int64_t pos, int window) {
    return (window > 0 && pos - window + 1 > 0) ? (int)(pos - window + 1) : 0;
}

// Shape checks shared by every entry point (no strides, no pointers).
int check_shape(int dtype, int T, int start_pos, int H, int KVH, int D, int window) {
    if (T < 1 || start_pos < 0 || H < 1 || KVH < 1 || D < 1 || window < 0) return PA_ERR_INVALID_ARG;
    if (H % KVH != 0) return PA_ERR_INVALID_ARG;
    if ((int64_t)start_pos + T > INT32_MAX) return PA_ERR_INVALID_ARG;
    if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16 && dtype != PA_DTYPE_F16) return PA_ERR_UNSUPPORTED;
    if (H / KVH > kRowsPerGroup) return PA_ERR_UNSUPPORTED;
    if (!find_variant(dtype, D)) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Splits along the keys when the grid would leave CUs idle: pick the split
// count whose longest-first schedule of (tile, split) items over the
// resident work-group slots finishes first, charging each extra split the
// cost of writing and merging its partial rows.
int choose_splits(const Variant &var, int T, int start_pos, int H, int KVH, int window,
                  int G, int TQ, int nq, int max_splits = kMaxSplits) {
    // a split's partial rows (written, then merged) cost about half a KV tile's
    // work when the query tile is full, proportionally less for short chunks
    const int rows = std::min(T, TQ) * G;
    const double split_cost = 0.5 * std::min(1.0, (double)rows / var.rows);
    const int slots = kCus * var.groups_per_cu;
    const int64_t base = (int64_t)nq * KVH;
    if (base >= slots) return 1;
    int64_t max_tiles = 0;
    for (int q = 0; q < nq; ++q) {
        const int t0 = q * TQ, tl = (int)std::min<int64_t>((int64_t)t0 + TQ, T) - 1;
        const int64_t kb = first_key_host((int64_t)start_pos + t0, window) / var.BK;
        const int64_t ke = ((int64_t)start_pos + tl) / var.BK + 1;
        max_tiles = std::max(max_tiles, ke - kb);
    }
    int best = 1;
    double best_cost = 1e300;
    for (int S = 1; S <= max_splits; ++S) {
        if (S > 1 && cdiv(max_tiles, S) < 4) break;
        const int64_t items = base * S;
        const double waves = (double)cdiv(items, slots);
        // one tile's time is the unit; a split adds a partial-row write+merge
        // of roughly half a tile for its work-group
        const double cost = waves * (double)cdiv(max_tiles, S) + (S > 1 ? split_cost * S : 0.0);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = S;
        }
    }
    (void)H;
    (void)G;
    return best;
}

int make_plan(int dtype, int T, int start_pos, int H, int KVH, int D, int window, Plan *pl,
              bool no_pack = false, int max_splits = kMaxSplits, bool mirror = false) {
    const int st = check_shape(dtype, T, start_pos, H, KVH, D, window);
    if (st != PA_OK) return st;
    const Variant *var = find_variant(dtype, D);
    // When full-size tiles cannot occupy every CU, work-groups that split each
    // tile's keys between their two wavefront halves (merged in LDS) come
    // before splitting the keys across work-groups (merged by a separate pass).
    if (const Variant *alt = find_ksplit_variant(dtype, D)) {
        const int64_t base = cdiv(T, var->rows / (H / KVH)) * KVH;
        if (base < (int64_t)kCus * var->groups_per_cu && alt->rows >= H / KVH) var = alt;
    }
    // The V operand-order copy costs a pass over the call's V rows and pays
    // off through their reuse by many query tiles; short chunks (decode,
    // draft verification) read V in place.
    // (a start_pos known only on the device also reads V in place: the copy
    // covers the call's tiles, which the host plan cannot know)
    // (with the caller's mirror of that copy only the new tiles are rewritten,
    // so the operand-order variant serves every chunk length)
    if (var->pack && !mirror && (no_pack || cdiv(T, var->rows / (H / KVH)) < kMinQueryTilesForPack))
        if (const Variant *alt = find_ksplit_variant(dtype, D, 0)) var = alt;
    pl->var = var;
    pl->G = H / KVH;
    pl->TQ = var->rows / pl->G;
    pl->nq = (int)cdiv(T, pl->TQ);
    pl->S = choose_splits(*var, T, start_pos, H, KVH, window, pl->G, pl->TQ, pl->nq, max_splits);
    // Causal tiles without a window and without key splits whose grid is
    // exactly one round of two work-groups per CU (nq * KVH = 512 with nq
    // even; at head_dim 128 with 16-bit inputs that is the 2048-token chunk of
    // 32 query heads over 8 kv heads): the long and the short query tile of a
    // kv head go into one work-group whose wavefront groups share the KV
    // tiles of the common key prefix (same rows per group, so the tile size
    // and the plan above stay valid), one such pair per CU.  On a smaller
    // grid the pair would only slow the long tile down; on a larger one (a
    // second round of work-groups) the fixed pairs lose to the dispatcher
    // refilling CUs as single tiles finish (measured on the 8192-token call).
    if (pl->S == 1 && pl->nq % 2 == 0 && (int64_t)pl->nq * KVH == 2 * (int64_t)kCus &&
        var->groups_per_cu == 2 && (window == 0 || (int64_t)window >= (int64_t)start_pos + T))
        if (const Variant *alt = find_ksplit_variant(dtype, D, 3))
            if (alt->rows == var->rows) var = pl->var = alt;
    const int64_t items = var->ksplit == 3 ? (int64_t)(pl->nq / 2) * KVH
                                           : (int64_t)pl->nq * KVH * pl->S;
    if (items > INT32_MAX) return PA_ERR_UNSUPPORTED;
    pl->items = (int)items;
    int64_t tiles = 0;
    for (int q = 0; q < pl->nq; ++q) {
        const int t0 = q * pl->TQ, tl = (int)std::min<int64_t>((int64_t)t0 + pl->TQ, T) - 1;
        const int64_t kb = first_key_host((int64_t)start_pos + t0, window) / var->BK;
        const int64_t ke = ((int64_t)start_pos + tl) / var->BK + 1;
        tiles += ke - kb;
    }
    pl->tiles = tiles * KVH;
    pl->vop_kt_lo = 0;
    pl->vop_tiles = 0;
    pl->vop_bytes = 0;
    pl->vmirror = nullptr;
    pl->pack0 = pl->npack = 0;
    if (var->pack && !mirror) {
        pl->vop_kt_lo = first_key_host(start_pos, window) / var->BK;
        pl->vop_tiles = (int)(((int64_t)start_pos + T - 1) / var->BK + 1 - pl->vop_kt_lo);
        const int64_t tile_bytes = (int64_t)var->BK * D * 2;
        if ((int64_t)pl->vop_tiles * tile_bytes > INT32_MAX) return PA_ERR_UNSUPPORTED;
        pl->vop_bytes = (size_t)(((int64_t)KVH * pl->vop_tiles * tile_bytes + 255) & ~(int64_t)255);
        pl->npack = pl->vop_tiles;
    }
    pl->ws_o_offset = pl->vop_bytes;
    pl->ws_ml_offset = pl->vop_bytes;
    pl->ws_bytes = pl->vop_bytes;
    if (pl->S > 1) {
        const size_t rows = (size_t)T * H;
        const size_t o_bytes = (size_t)pl->S * rows * D * sizeof(float);
        pl->ws_ml_offset = pl->ws_o_offset + ((o_bytes + 255) & ~(size_t)255);
        pl->ws_bytes = pl->ws_ml_offset + (size_t)pl->S * rows * sizeof(float2);
    }
    return PA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// Where key j of a kv head lives: row j (linear), slot j % ring (ring > 0),
// or page page_table[j >> page_shift] of a pool of num_pages pages (paged).
struct CacheLayout {
    int ring = 0;
    const int32_t *page_table = nullptr;
    int page_shift = 0, num_pages = 0;
    const int32_t *start_pos_dev = nullptr;   // start_pos read by the kernels (planned for the max)
};

int launch(const Plan &pl, int dtype, const void *q, int64_t q_row_stride, const void *k,
           const void *v, int64_t kv_head_stride, const CacheLayout &lay, void *out,
           int64_t out_row_stride, int out_dtype, int T, int start_pos, int H, int KVH, int D, int window, void *ws,
           hipStream_t stream) {
    const int ring = lay.ring;
    Params p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.out_dtype = out_dtype;
    p.ws_o = pl.S > 1 ? (float *)((char *)ws + pl.ws_o_offset) : nullptr;
    p.ws_ml = pl.S > 1 ? (float2 *)((char *)ws + pl.ws_ml_offset) : nullptr;
    uint16_t *const vop = pl.var->pack ? (uint16_t *)(pl.vmirror ? pl.vmirror : ws) : nullptr;
    p.vop = vop;
    p.vop_kt_lo = pl.vop_kt_lo;
    p.vop_tiles = pl.vop_tiles;
    p.vop_pack0 = pl.pack0;
    p.q_row_stride = q_row_stride;
    p.kv_head_stride = kv_head_stride;
    p.out_row_stride = out_row_stride;
    p.T = T;
    p.start_pos = start_pos;
    p.H = H;
    p.KVH = KVH;
    p.G = pl.G;
    p.window = window;
    p.TQ = pl.TQ;
    p.nq = pl.nq;
    p.S = pl.S;
    p.n_items = pl.items;
    p.c = (float)(1.4426950408889634 / sqrt((double)D));
    p.order = pl.var->groups_per_cu == 2 ? 1 : 0;
    p.pair = pl.var->ksplit == 3;
    p.L = start_pos + T;
    p.ring = ring;
    p.page_table = lay.page_table;
    p.page_shift = lay.page_shift;
    p.num_pages = lay.num_pages;
    p.start_pos_dev = lay.start_pos_dev;
    p.kv_bytes = (int)std::min<int64_t>((ring ? (int64_t)ring : (int64_t)start_pos + T) * D *
                                            elem_bytes(dtype), INT32_MAX);
    if (pl.var->pack && pl.npack > 0) {
        hipLaunchKernelGGL(pl.var->pack, dim3(pl.npack, KVH), dim3(256), 0, stream, p, vop);
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    }
    const KernelFn fn = lay.page_table ? pl.var->fn_paged : ring ? pl.var->fn_ring : pl.var->fn;
    hipLaunchKernelGGL(fn, dim3(pl.items), dim3(pl.var->threads), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    if (pl.S > kWideMergeSplits) {
        hipLaunchKernelGGL(wide_merge_for(D), dim3((unsigned)((int64_t)T * H)), dim3(512), 0, stream,
                           (const float *)p.ws_o, (const float2 *)p.ws_ml, out, out_dtype,
                           out_row_stride, T, H, pl.S);
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    } else if (pl.S > 1) {
        const int64_t n = (int64_t)T * H * (D / 4);
        hipLaunchKernelGGL(merge_for(D), dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream,
                           (const float *)p.ws_o, (const float2 *)p.ws_ml, out, out_dtype,
                           out_row_stride, T, H, pl.S, p.c);
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    }
    return PA_OK;
}

// rows_per_head: the rows the kernels address in each kv head's block (L for
// a linear cache, the slot count of a ring).
int check_args(int dtype, const void *q, int64_t q_row_stride, const void *k, const void *v,
               int64_t kv_head_stride, int64_t rows_per_head, const void *out,
               int64_t out_row_stride, int out_dtype, int T, int start_pos, int H, int KVH, int D,
               int window) {
    if (!q || !k || !v || !out) return PA_ERR_INVALID_ARG;
    const int st = check_shape(dtype, T, start_pos, H, KVH, D, window);
    if (st == PA_ERR_INVALID_ARG) return st;
    const int64_t row = (int64_t)H * D;
    if (q_row_stride < row || out_row_stride < row) return PA_ERR_INVALID_ARG;
    if (kv_head_stride < rows_per_head * D) return PA_ERR_INVALID_ARG;
    if (st != PA_OK) return st;
    const int eb = elem_bytes(dtype);
    // the 16-bit kernels address one kv head's rows with 32-bit buffer offsets
    if (dtype != PA_DTYPE_F32 && rows_per_head * D * eb > kMaxHeadBytes) return PA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PA_ERR_UNSUPPORTED;
    if (out_dtype != PA_DTYPE_F32 && out_dtype != PA_DTYPE_BF16 && out_dtype != PA_DTYPE_F16)
        return PA_ERR_UNSUPPORTED;
    // outputs go out in groups of four elements of a row (16 or 8 bytes)
    if ((q_row_stride * eb) % 16 || (kv_head_stride * eb) % 16 || out_row_stride % 4)
        return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Scratch of the packed entry points: one buffer per (device, stream), so
// that calls on different streams never share one, grown on demand.  The
// lock is held from the lookup through the launch: a call that grows a
// buffer first waits for the work already enqueued on its stream (the only
// work that can use it) and no other thread can hold the old pointer.
struct StreamScratch {
    int dev;
    hipStream_t stream;
    void *ptr;
    size_t bytes;
};
std::mutex g_scratch_mutex;
std::vector<StreamScratch> g_scratch;

// Called with g_scratch_mutex held.
int scratch_for(size_t need, hipStream_t stream, void **out) {
    *out = nullptr;
    if (need == 0) return PA_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    StreamScratch *s = nullptr;
    for (StreamScratch &e : g_scratch)
        if (e.dev == dev && e.stream == stream) s = &e;
    if (!s) {
        g_scratch.push_back(StreamScratch{dev, stream, nullptr, 0});
        s = &g_scratch.back();
    }
    if (s->bytes < need) {
        if (s->ptr) {
            // work already enqueued on this stream may still read the old buffer
            if (hipStreamSynchronize(stream) != hipSuccess) return PA_ERR_HIP;
            if (hipFree(s->ptr) != hipSuccess) return PA_ERR_HIP;
            s->ptr = nullptr;
            s->bytes = 0;
        }
        const size_t grow = need + need / 4;
        if (hipMalloc(&s->ptr, grow) != hipSuccess) {
            s->ptr = nullptr;
            return PA_ERR_HIP;
        }
        s->bytes = grow;
    }
    *out = s->ptr;
    return PA_OK;
}

int run_packed(int dtype, const void *q, const void *k, const void *v, float *out, int T,
               int start_pos, int H, int KVH, int D, int window, void *stream) {
    const int64_t row = (int64_t)H * D;
    const int64_t kvs = ((int64_t)start_pos + T) * D;
    int st = check_args(dtype, q, row, k, v, kvs, (int64_t)start_pos + T, out, row, PA_DTYPE_F32, T,
                        start_pos, H, KVH, D, window);
    if (st != PA_OK) return st;
    Plan pl;
    st = make_plan(dtype, T, start_pos, H, KVH, D, window, &pl);
    if (st != PA_OK) return st;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    void *ws = nullptr;
    st = scratch_for(pl.ws_bytes, (hipStream_t)stream, &ws);
    if (st != PA_OK) return st;
    return launch(pl, dtype, q, row, k, v, kvs, CacheLayout{}, out, row, PA_DTYPE_F32, T, start_pos,
                  H, KVH, D, window, ws, (hipStream_t)stream);
}

// Plan, workspace check and launch of the strided entry points (arguments checked).
int run_ex(int dtype, const void *q, int64_t q_row_stride, const void *k, const void *v,
           int64_t kv_head_stride, const CacheLayout &lay, void *out, int64_t out_row_stride,
           int out_dtype, int T, int start_pos, int H, int KVH, int D, int window, void *workspace,
           size_t workspace_bytes, void *stream) {
    Plan pl;
    const int st = make_plan(dtype, T, start_pos, H, KVH, D, window, &pl, lay.start_pos_dev != nullptr);
    if (st != PA_OK) return st;
    if (pl.ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl.ws_bytes) return PA_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255) != 0) return PA_ERR_WORKSPACE;
    }
    return launch(pl, dtype, q, q_row_stride, k, v, kv_head_stride, lay, out, out_row_stride, out_dtype, T,
                  start_pos, H, KVH, D, window, workspace, (hipStream_t)stream);
}

}  // namespace

// ---- scratch without allocation ------------------------------------------------------
//
// prefill_attn_noalloc_ex keeps its workspace (split partials, the V copy) in
// this array instead of memory the library allocates or the caller passes:
// each GPU the library runs on holds one copy of it until the process ends.
// Host code never uses the array's name as an address: the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device on
// the entry point's first call there (with that device current).  Nothing in
// it has to start at zero: every byte a call reads was written earlier in the
// same call.

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mutex;
void *g_noalloc_ptr[kMaxDevices];

// This device's copy of `scratch` (device address), or PA_ERR_HIP.
int noalloc_scratch(void **out) {
    *out = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_noalloc_mutex);
    if (!g_noalloc_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_HIP;
        g_noalloc_ptr[dev] = ptr;
    }
    *out = g_noalloc_ptr[dev];
    return PA_OK;
}

}  // namespace

// ---- C ABI -----------------------------------------------------------------------------

extern "C" {

int prefill_attn_f32(const float *q, const float *k_cache, const float *v_cache, float *out, int T,
                     int start_pos, int num_heads, int num_kv_heads, int head_dim, int window,
                     void *stream) {
    return run_packed(PA_DTYPE_F32, q, k_cache, v_cache, out, T, start_pos, num_heads,
                      num_kv_heads, head_dim, window, stream);
}

int prefill_attn_bf16(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                      float *out, int T, int start_pos, int num_heads, int num_kv_heads,
                      int head_dim, int window, void *stream) {
    return run_packed(PA_DTYPE_BF16, q, k_cache, v_cache, out, T, start_pos, num_heads,
                      num_kv_heads, head_dim, window, stream);
}

int prefill_attn_f16(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                     float *out, int T, int start_pos, int num_heads, int num_kv_heads,
                     int head_dim, int window, void *stream) {
    return run_packed(PA_DTYPE_F16, q, k_cache, v_cache, out, T, start_pos, num_heads,
                      num_kv_heads, head_dim, window, stream);
}

int prefill_attn_ex(int dtype, const void *q, int64_t q_row_stride, const void *k_cache,
                    const void *v_cache, int64_t kv_head_stride, void *out,
                    int64_t out_row_stride, int out_dtype, int T, int start_pos, int num_heads,
                    int num_kv_heads, int head_dim, int window, void *workspace,
                    size_t workspace_bytes, void *stream) {
    int st = check_args(dtype, q, q_row_stride, k_cache, v_cache, kv_head_stride,
                        (int64_t)start_pos + T, out, out_row_stride, out_dtype, T, start_pos, num_heads,
                        num_kv_heads, head_dim, window);
    if (st != PA_OK) return st;
    return run_ex(dtype, q, q_row_stride, k_cache, v_cache, kv_head_stride, CacheLayout{}, out,
                  out_row_stride, out_dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window, workspace,
                  workspace_bytes, stream);
}

size_t prefill_attn_vmirror_bytes(int dtype, int num_kv_heads, int head_dim, int capacity) {
    if (num_kv_heads < 1 || capacity < 1) return 0;
    const Variant *var = find_variant(dtype, head_dim);
    if (!var || !var->pack) return 0;
    // one kv head's tiles are addressed with 32-bit buffer offsets
    const int64_t per_head = cdiv(capacity, var->BK) * var->BK * head_dim * 2;
    if (per_head > kMaxHeadBytes) return 0;
    return (size_t)num_kv_heads * (size_t)per_head;
}

int prefill_attn_vmirror_ex(int dtype, const void *q, int64_t q_row_stride, const void *k_cache,
                            const void *v_cache, int64_t kv_head_stride, void *v_mirror,
                            int mirror_capacity, int mirror_keys, void *out, int64_t out_row_stride,
                            int out_dtype, int T, int start_pos, int num_heads, int num_kv_heads,
                            int head_dim, void *workspace, size_t workspace_bytes, void *stream) {
    const int64_t L = (int64_t)start_pos + T;
    int st = check_args(dtype, q, q_row_stride, k_cache, v_cache, kv_head_stride, L, out,
                        out_row_stride, out_dtype, T, start_pos, num_heads, num_kv_heads, head_dim, 0);
    if (st != PA_OK) return st;
    // no kernel of this dtype and head_dim reads V in operand order: the
    // mirror plays no part (prefill_attn_ex with window 0)
    if (!find_variant(dtype, head_dim)->pack)
        return run_ex(dtype, q, q_row_stride, k_cache, v_cache, kv_head_stride, CacheLayout{}, out,
                      out_row_stride, out_dtype, T, start_pos, num_heads, num_kv_heads, head_dim, 0,
                      workspace, workspace_bytes, stream);
    if (!v_mirror || mirror_capacity < L || mirror_keys < 0 || mirror_keys > L) return PA_ERR_INVALID_ARG;
    if (!aligned16(v_mirror) || prefill_attn_vmirror_bytes(dtype, num_kv_heads, head_dim, mirror_capacity) == 0)
        return PA_ERR_UNSUPPORTED;
    Plan pl;
    st = make_plan(dtype, T, start_pos, num_heads, num_kv_heads, head_dim, 0, &pl, false, kMaxSplits, true);
    if (st != PA_OK) return st;
    if (!pl.var->pack) return PA_ERR_UNSUPPORTED;
    const int BK = pl.var->BK;
    pl.vmirror = v_mirror;
    pl.vop_kt_lo = 0;
    pl.vop_tiles = (int)cdiv(mirror_capacity, BK);
    // from the tile of the first key the mirror lacks through the call's last
    // tile, which is always rewritten (its keys past L become zeros)
    pl.pack0 = (int)(std::min<int64_t>(mirror_keys, L - 1) / BK);
    pl.npack = (int)(cdiv(L, BK) - pl.pack0);
    if (pl.ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl.ws_bytes) return PA_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255) != 0) return PA_ERR_WORKSPACE;
    }
    return launch(pl, dtype, q, q_row_stride, k_cache, v_cache, kv_head_stride, CacheLayout{}, out,
                  out_row_stride, out_dtype, T, start_pos, num_heads, num_kv_heads, head_dim, 0, workspace,
                  (hipStream_t)stream);
}

int prefill_attn_noalloc_ex(int dtype, const void *q, int64_t q_row_stride, const void *k_cache,
                            const void *v_cache, int64_t kv_head_stride, void *out,
                            int64_t out_row_stride, int out_dtype, int T, int start_pos,
                            int num_heads, int num_kv_heads, int head_dim, int window, void *stream) {
    int st = check_args(dtype, q, q_row_stride, k_cache, v_cache, kv_head_stride,
                        (int64_t)start_pos + T, out, out_row_stride, out_dtype, T, start_pos, num_heads,
                        num_kv_heads, head_dim, window);
    if (st != PA_OK) return st;
    // prefill_attn_ex's plan when its workspace fits the array; otherwise V
    // read in place and the fewest fewer key splits whose partials fit (one
    // split needs none)
    Plan pl;
    st = make_plan(dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window, &pl);
    if (st == PA_OK && pl.ws_bytes > PA_NOALLOC_SCRATCH_BYTES) {
        st = make_plan(dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window, &pl, true);
        while (st == PA_OK && pl.ws_bytes > PA_NOALLOC_SCRATCH_BYTES && pl.S > 1)
            st = make_plan(dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window, &pl, true,
                           pl.S - 1);
    }
    if (st != PA_OK) return st;
    if (pl.ws_bytes > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (pl.ws_bytes > 0) {
        st = noalloc_scratch(&ws);
        if (st != PA_OK) return st;
    }
    return launch(pl, dtype, q, q_row_stride, k_cache, v_cache, kv_head_stride, CacheLayout{}, out,
                  out_row_stride, out_dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window,
                  ws, (hipStream_t)stream);
}

int prefill_attn_ring_ex(int dtype, const void *q, int64_t q_row_stride, const void *k_ring,
                         const void *v_ring, int64_t kv_head_stride, int ring_slots, void *out,
                         int64_t out_row_stride, int out_dtype, int T, int start_pos, int num_heads,
                         int num_kv_heads, int head_dim, int window, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (ring_slots < 1) return PA_ERR_INVALID_ARG;
    int st = check_args(dtype, q, q_row_stride, k_ring, v_ring, kv_head_stride, ring_slots, out,
                        out_row_stride, out_dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window);
    if (st != PA_OK) return st;
    // the ring must hold every key the chunk reads at once: the window before
    // the chunk's first query through its last key
    const int64_t L = (int64_t)start_pos + T;
    const int64_t need = window > 0 ? std::min<int64_t>(L, (int64_t)window + T - 1) : L;
    if (ring_slots < need) return PA_ERR_INVALID_ARG;
    // a ring at least as long as the call is a linear cache (slot j holds key j)
    CacheLayout lay;
    lay.ring = ring_slots >= L ? 0 : (int)ring_slots;
    return run_ex(dtype, q, q_row_stride, k_ring, v_ring, kv_head_stride, lay, out, out_row_stride,
                  out_dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window, workspace,
                  workspace_bytes, stream);
}

int prefill_attn_paged_dev_ex(int dtype, const void *q, int64_t q_row_stride, const void *k_pool,
                              const void *v_pool, int page_size, int num_pages,
                              const int32_t *page_table, void *out, int64_t out_row_stride,
                              int out_dtype, int T, const int32_t *start_pos_dev, int max_start_pos, int num_heads,
                              int num_kv_heads, int head_dim, int window, void *workspace,
                              size_t workspace_bytes, void *stream) {
    if (!start_pos_dev) return PA_ERR_INVALID_ARG;
    if (!page_table || num_pages < 1) return PA_ERR_INVALID_ARG;
    if (page_size < 64 || (page_size & (page_size - 1)) != 0) return PA_ERR_UNSUPPORTED;
    int st = check_args(dtype, q, q_row_stride, k_pool, v_pool, (int64_t)page_size * head_dim,
                        page_size, out, out_row_stride, out_dtype, T, max_start_pos, num_heads, num_kv_heads,
                        head_dim, window);
    if (st != PA_OK) return st;
    CacheLayout lay;
    lay.page_table = page_table;
    lay.page_shift = __builtin_ctz((unsigned)page_size);
    lay.num_pages = num_pages;
    lay.start_pos_dev = start_pos_dev;
    return run_ex(dtype, q, q_row_stride, k_pool, v_pool, 0, lay, out, out_row_stride, out_dtype, T,
                  max_start_pos, num_heads, num_kv_heads, head_dim, window, workspace,
                  workspace_bytes, stream);
}

int prefill_attn_paged_ex(int dtype, const void *q, int64_t q_row_stride, const void *k_pool,
                          const void *v_pool, int page_size, int num_pages,
                          const int32_t *page_table, void *out, int64_t out_row_stride,
                          int out_dtype, int T, int start_pos, int num_heads, int num_kv_heads, int head_dim, int window,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (!page_table || num_pages < 1) return PA_ERR_INVALID_ARG;
    // a page holds whole KV tiles of every kernel (64 keys at most)
    if (page_size < 64 || (page_size & (page_size - 1)) != 0) return PA_ERR_UNSUPPORTED;
    // the pool's pages as the head stride of a linear cache of num_pages*page_size
    // rows: the shape and pointer checks are those of prefill_attn_ex
    int st = check_args(dtype, q, q_row_stride, k_pool, v_pool, (int64_t)page_size * head_dim,
                        page_size, out, out_row_stride, out_dtype, T, start_pos, num_heads, num_kv_heads,
                        head_dim, window);
    if (st != PA_OK) return st;
    CacheLayout lay;
    lay.page_table = page_table;
    lay.page_shift = __builtin_ctz((unsigned)page_size);
    lay.num_pages = num_pages;
    return run_ex(dtype, q, q_row_stride, k_pool, v_pool, 0, lay, out, out_row_stride, out_dtype, T,
                  start_pos,
                  num_heads, num_kv_heads, head_dim, window, workspace, workspace_bytes, stream);
}

int prefill_kv_write(int dtype, const void *k_src, const void *v_src, int64_t src_row_stride,
                     void *k_cache, void *v_cache, int64_t kv_head_stride, int ring_slots, int T,
                     int start_pos, int num_kv_heads, int head_dim, void *stream) {
    if (!k_src || !v_src || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
    if (T < 1 || start_pos < 0 || num_kv_heads < 1 || head_dim < 1 || ring_slots < 0)
        return PA_ERR_INVALID_ARG;
    if ((int64_t)start_pos + T > INT32_MAX) return PA_ERR_INVALID_ARG;
    if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16 && dtype != PA_DTYPE_F16)
        return PA_ERR_UNSUPPORTED;
    const int64_t rows = ring_slots ? ring_slots : (int64_t)start_pos + T;
    if (src_row_stride < (int64_t)num_kv_heads * head_dim) return PA_ERR_INVALID_ARG;
    if (kv_head_stride < rows * head_dim) return PA_ERR_INVALID_ARG;
    const int eb = elem_bytes(dtype);
    const int64_t row_bytes = (int64_t)head_dim * eb;
    if (row_bytes % 16 || (src_row_stride * eb) % 16 || (kv_head_stride * eb) % 16)
        return PA_ERR_UNSUPPORTED;
    if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_UNSUPPORTED;
    // tokens a later token of the chunk overwrites in a ring are skipped
    const int t_first = ring_slots && T > ring_slots ? T - ring_slots : 0;
    const int64_t chunks = 2 * (int64_t)(T - t_first) * num_kv_heads * (row_bytes / 16);
    if (chunks > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(chunks, 256), 8 * kCus);
    hipLaunchKernelGGL(kv_write, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t *)k_src, (const uint8_t *)v_src, src_row_stride * eb,
                       (uint8_t *)k_cache, (uint8_t *)v_cache, kv_head_stride * eb, (int)row_bytes,
                       num_kv_heads, t_first, T, start_pos, ring_slots);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t prefill_attn_workspace_bytes(int dtype, int T, int start_pos, int num_heads,
                                    int num_kv_heads, int head_dim, int window) {
    Plan pl;
    if (make_plan(dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window, &pl) != PA_OK)
        return 0;
    return pl.ws_bytes;
}

int prefill_attn_plan(int dtype, int T, int start_pos, int num_heads, int num_kv_heads,
                      int head_dim, int window, int64_t *info, int n) {
    Plan pl;
    const int st = make_plan(dtype, T, start_pos, num_heads, num_kv_heads, head_dim, window, &pl);
    if (st != PA_OK) return st;
    const int64_t vals[8] = {pl.TQ, pl.nq, pl.S, pl.items, pl.var->BK, pl.var->threads / kWave,
                             (int64_t)pl.ws_bytes, pl.tiles};
    for (int i = 0; i < n && i < 8 && info; ++i) info[i] = vals[i];
    return PA_OK;
}

const char *prefill_attn_strerror(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported head_dim, dtype, group size or alignment";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    }
    return "unknown status";
}

}  // extern "C"
