/*
 * prefill_attn.h -- C ABI of the MI355X (gfx950) chunked causal grouped-query
 * prefill attention library, libprefill_attn.so.
 *
 * The operation (gnosis handoff page "Prefill attention -> GPU: handoff",
 * section "GPU design (the real fix)"):
 *
 *   A chunk of T query tokens, at sequence positions start_pos .. start_pos+T-1,
 *   attends to the L = start_pos + T keys held in a KV cache.  Query head h
 *   uses kv head h / (num_heads / num_kv_heads) (grouped-query attention).
 *   For query token t (position pos = start_pos + t) and each valid key j:
 *       s_j = (q_t . k_j) / sqrt(head_dim)
 *   valid keys are j <= pos (causal mask, Step 2 of that section) and, when
 *   window > 0, j >= pos - window + 1 (the per-row contiguous band of the
 *   TensorSharp page "Design: closing the Gemma-4 long-prompt prefill gap",
 *   section 5, Option A: `window` keys including the query's own).  The row
 *   softmax of the valid scores weights the value rows:
 *       out_t = sum_j softmax(s)_j * v_j                      (Step 3)
 *   Masked keys contribute exactly nothing.  window <= 0 means no window.
 *   Keys that no row of the call reads (below the first query's window
 *   start, and at or past L) never reach out: the kernels skip them or load
 *   them as zeros, so those cache rows may hold anything, NaN included.  A
 *   non-finite value at a key that some row reads makes that row's output
 *   non-finite, as the definition does; since the query rows of one kv head
 *   that are computed together (up to 128 (token, head) rows) share each K/V
 *   tile, it can also reach the other rows of that group.
 *
 * Layouts (all element offsets, row-major; same page, "Layout"):
 *   q        (t, h, d)  at q[t*q_row_stride + h*head_dim + d]
 *            packed entry points: q_row_stride = num_heads*head_dim (the
 *            page's qkv_dim)
 *   k_cache, v_cache
 *            (kh, j, d) at k_cache[kh*kv_head_stride + j*head_dim + d],
 *            one contiguous [L x head_dim] block per kv head; packed entry
 *            points: kv_head_stride = L*head_dim.  A cache allocated for
 *            `capacity` positions passes kv_head_stride = capacity*head_dim
 *            to prefill_attn_ex; rows L .. capacity-1 are never read, so
 *            they may hold anything, NaN included.
 *   out      (t, h, d)  at out[t*out_row_stride + h*head_dim + d];
 *            packed entry points: out_row_stride = num_heads*head_dim.
 *
 * Storage types: fp32, bf16 or fp16 for q/k/v (bf16 and fp16 passed as
 * uint16_t bit patterns).  out is fp32 (the page's bf16 workload keeps an
 * fp32 output; the packed entry points always write fp32); the strided forms
 * take out_dtype, a PA_DTYPE_* value, and then write the fp32 result rounded
 * to the nearest even bf16 or fp16 for a caller whose next step reads 16-bit
 * activations.  bf16/fp16 inputs are multiplied on the matrix cores with fp32
 * accumulation; the softmax runs in fp32.
 *
 * Supported shapes: head_dim in {32, 64, 128, 256, 512} for bf16/fp16 and
 * {32, 64, 128, 256} for fp32; any T >= 1, start_pos >= 0, num_heads a
 * multiple of num_kv_heads with num_heads/num_kv_heads <= 128.  Pointers must
 * be 16-byte aligned, q_row_stride and kv_head_stride must keep every row
 * 16-byte aligned and out_row_stride must be a multiple of 4 elements.
 *
 * Ownership: every pointer is caller-owned device memory.  The library keeps
 * no pointer after a call returns, never frees caller memory, only reads q,
 * k_cache and v_cache, and writes every element (t, h, d) of out (nothing
 * else in out's rows).
 *
 * Errors: arguments are checked before anything is enqueued; a violation
 * returns PA_ERR_INVALID_ARG (or PA_ERR_UNSUPPORTED for a shape or alignment
 * the library has no kernel for) and leaves out untouched.  A failed launch
 * returns PA_ERR_HIP.  Calls are asynchronous on `stream` (a hipStream_t,
 * NULL for the null stream): faults inside a kernel surface at the caller's
 * next synchronisation, as usual for HIP.  No C++ exception crosses this
 * interface.
 */
#ifndef PREFILL_ATTN_H
#define PREFILL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PA_OK 0
#define PA_ERR_INVALID_ARG 1   /* null pointer, T < 1, start_pos < 0, heads < 1,
                                  num_heads % num_kv_heads != 0, window < 0,
                                  a stride below its minimum                      */
#define PA_ERR_UNSUPPORTED 2   /* head_dim, dtype, out_dtype, group size or
                                  alignment                                       */
#define PA_ERR_HIP 3           /* a HIP runtime call or launch failed             */
#define PA_ERR_WORKSPACE 4     /* workspace missing or smaller than required      */

/* storage types of q, k_cache and v_cache */
#define PA_DTYPE_F32 0
#define PA_DTYPE_BF16 1
#define PA_DTYPE_F16 2

/*
 * Packed entry points: q [T][num_heads][head_dim], caches
 * [num_kv_heads][L][head_dim] with L = start_pos + T, out [T][num_heads][head_dim].
 * Scratch memory (bf16/fp16 inputs at head_dim 512: a copy of the call's V
 * rows rearranged into matrix-core operand order; every dtype: split-KV
 * partial results when the keys are split) comes from a buffer per (device,
 * stream) that the library allocates on first need and grows (hipMalloc;
 * growing first waits for the work already enqueued on that stream, the only
 * work that can use the old buffer).  Calls from several host threads are
 * safe (a lock covers the lookup and the launch), and calls on different
 * streams never share a buffer.  Buffers live until the process ends.
 */
int prefill_attn_f32(const float *q, const float *k_cache, const float *v_cache, float *out,
                     int T, int start_pos, int num_heads, int num_kv_heads, int head_dim,
                     int window, void *stream);
int prefill_attn_bf16(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                      float *out, int T, int start_pos, int num_heads, int num_kv_heads,
                      int head_dim, int window, void *stream);
int prefill_attn_f16(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                     float *out, int T, int start_pos, int num_heads, int num_kv_heads,
                     int head_dim, int window, void *stream);

/*
 * General form: explicit strides (in elements) and an explicit workspace.
 * dtype is a PA_DTYPE_* value, the storage type of q, k_cache and v_cache;
 * out_dtype, a PA_DTYPE_* value too, is out's (any of the three with any
 * dtype; the split-KV partials in the workspace stay fp32 whatever it is).
 * workspace may be NULL when
 * prefill_attn_workspace_bytes() returns 0 for the same arguments; otherwise
 * it must be device memory of at least that many bytes, 256-byte aligned,
 * and it must not be used by anything else until the work enqueued by this
 * call has finished.  Nothing is allocated.
 */
int prefill_attn_ex(int dtype, const void *q, int64_t q_row_stride,
                    const void *k_cache, const void *v_cache, int64_t kv_head_stride,
                    void *out, int64_t out_row_stride, int out_dtype,
                    int T, int start_pos, int num_heads, int num_kv_heads, int head_dim,
                    int window, void *workspace, size_t workspace_bytes, void *stream);

/*
 * prefill_attn_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc)
 * and have no workspace to pass: the same arguments without the workspace.
 * Its scratch is a fixed array of PA_NOALLOC_SCRATCH_BYTES in device memory,
 * one per GPU, held from the library's first use on that GPU until the
 * process ends; nothing is allocated or freed by the call.  When the plan
 * prefill_attn_ex would use fits in it, that plan runs (same kernels, same
 * result bits); otherwise V is read in place and the keys are split fewer
 * times, down to a plan that needs no scratch, so no size is refused for the
 * scratch's sake (PA_ERR_WORKSPACE would mean it could not fit, which no
 * plan reaches).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams, or different threads
 * without ordering) race on it and must not be issued; calls ordered on one
 * stream are fine.  Errors as for prefill_attn_ex, plus PA_ERR_HIP when the
 * array's device address cannot be obtained.
 */
#define PA_NOALLOC_SCRATCH_BYTES 33554432   /* 32 MiB */
int prefill_attn_noalloc_ex(int dtype, const void *q, int64_t q_row_stride,
                            const void *k_cache, const void *v_cache, int64_t kv_head_stride,
                            void *out, int64_t out_row_stride, int out_dtype,
                            int T, int start_pos, int num_heads, int num_kv_heads, int head_dim,
                            int window, void *stream);

/*
 * prefill_attn_ex without a window, for the chunks of one long sequence in
 * turn (the TensorSharp page "Design: closing the Gemma-4 long-prompt prefill
 * gap", section 2: the head_dim 512 global layers prefilled as 2048-token
 * chunks over tens of thousands of cached keys), with a mirror of V that the
 * caller keeps.  At head_dim 512 with bf16/fp16 inputs the kernels read V in
 * matrix-core operand order; prefill_attn_ex rewrites every V row the call
 * reads into that order in its workspace on every call (a pass over the whole
 * cache per chunk).  Here the rewritten tiles live in v_mirror across calls
 * and each call rewrites only the keys the mirror lacks.
 *   v_mirror         device memory of prefill_attn_vmirror_bytes(dtype,
 *                    num_kv_heads, head_dim, mirror_capacity) bytes, 16-byte
 *                    aligned, owned by the caller; its layout is the
 *                    library's own (tiles of keys in operand order per kv head)
 *   mirror_capacity  keys it can hold (>= start_pos + T)
 *   mirror_keys      keys 0 .. mirror_keys-1 that it already holds: written
 *                    by earlier calls of this function for the same v_cache,
 *                    whose rows 0 .. mirror_keys-1 have not changed since
 *                    (0 <= mirror_keys <= start_pos + T; 0 rewrites all)
 * After the call's work has run, the mirror holds keys 0 .. start_pos+T-1, so
 * the next chunk of the sequence passes mirror_keys = start_pos + T.  Calls
 * that use one mirror must be ordered (one stream, or synchronised), as must
 * any work that writes the rows of v_cache the mirror holds.  The result bits
 * are those of prefill_attn_ex for the same arguments whenever that call
 * rewrites V too (at least 8 query tiles); for shorter chunks, which it runs
 * on V in place, they agree to rounding.  The workspace is the one
 * prefill_attn_workspace_bytes gives for the same arguments (an upper
 * bound: the V copy it counts is not used).  For a dtype and head_dim whose
 * kernels read V in place (prefill_attn_vmirror_bytes returns 0) the call is
 * prefill_attn_ex with window 0 and v_mirror is not touched.  Errors as for
 * prefill_attn_ex, plus PA_ERR_INVALID_ARG for a null v_mirror,
 * mirror_capacity < start_pos + T or mirror_keys outside [0, start_pos + T],
 * and PA_ERR_UNSUPPORTED for a misaligned v_mirror or a capacity whose
 * mirror has no size (see below).
 */
int prefill_attn_vmirror_ex(int dtype, const void *q, int64_t q_row_stride,
                            const void *k_cache, const void *v_cache, int64_t kv_head_stride,
                            void *v_mirror, int mirror_capacity, int mirror_keys,
                            void *out, int64_t out_row_stride, int out_dtype,
                            int T, int start_pos, int num_heads, int num_kv_heads, int head_dim,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of the V mirror prefill_attn_vmirror_ex reads for `capacity` keys;
 * 0 when no kernel of this dtype and head_dim reads one (then the mirror is
 * not needed), for invalid arguments, and when one kv head's share would
 * pass 2 GiB.
 */
size_t prefill_attn_vmirror_bytes(int dtype, int num_kv_heads, int head_dim, int capacity);

/*
 * Ring cache form (sliding-window layers).  The TensorSharp page "Design:
 * closing the Gemma-4 long-prompt prefill gap", section 4, requirement R4,
 * has sliding-window layers write the K/V of position pos into slot
 * pos % (ring size) of a circular cache instead of row pos.  Here key j of
 * kv head kh is read from
 *     k_ring[kh*kv_head_stride + (j % ring_slots)*head_dim + d]   (v_ring alike)
 * and everything else is prefill_attn_ex.  The caller has written the
 * chunk's own keys before the call, so every key the chunk reads must be
 * resident at once: ring_slots >= min(L, window + T - 1) for window > 0 and
 * ring_slots >= L for window 0 (a ring that short cannot hold them and the
 * call returns PA_ERR_INVALID_ARG; for T = 1, window slots suffice).  Slots
 * that hold no key of [0, L) are never read, so they may hold anything,
 * NaN included.  kv_head_stride >= ring_slots*head_dim.  The workspace is
 * the one prefill_attn_workspace_bytes gives for the same shape.
 */
int prefill_attn_ring_ex(int dtype, const void *q, int64_t q_row_stride,
                         const void *k_ring, const void *v_ring, int64_t kv_head_stride,
                         int ring_slots, void *out, int64_t out_row_stride, int out_dtype,
                         int T, int start_pos, int num_heads, int num_kv_heads, int head_dim,
                         int window, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Paged cache form (short chunks and decode over a shared pool; the FreeToken
 * page "perf(spec): capture the gemma4 assistant draft in cuda graphs": each
 * draft step reads the sequence's [0, cached_len) keys through its page
 * table).  k_pool and v_pool hold num_pages pages; page pg holds page_size
 * consecutive positions of every kv head:
 *     k_pool[((pg*num_kv_heads + kh)*page_size + r)*head_dim + d]   (v_pool alike)
 * and key j of kv head kh is row j % page_size of page page_table[j / page_size].
 * page_table is device memory (int32) with at least ceil(L / page_size)
 * entries; it is read by the kernels, so it may be rewritten between calls
 * (e.g. inside a captured graph's fixed buffer).  page_size must be a power
 * of two >= 64 (every KV tile then lies in one page).  Entries of blocks that
 * no row reads (below every row's window) may hold anything; an entry outside
 * [0, num_pages) reads as zeros (no fault).  Everything else is
 * prefill_attn_ex, including the workspace it needs for the same shape.
 */
int prefill_attn_paged_ex(int dtype, const void *q, int64_t q_row_stride,
                          const void *k_pool, const void *v_pool, int page_size, int num_pages,
                          const int32_t *page_table, void *out, int64_t out_row_stride,
                          int out_dtype, int T, int start_pos, int num_heads, int num_kv_heads, int head_dim,
                          int window, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The paged form with start_pos in device memory: *start_pos_dev (int32,
 * read by the kernels when they run) replaces start_pos, so one captured
 * graph serves every length of a decode or draft loop (the FreeToken page
 * copies the cached length into a fixed buffer before each replay).  The
 * launch is planned for max_start_pos, which bounds the device value (larger
 * values are clamped to it, negative ones to 0); the workspace is the one
 * prefill_attn_workspace_bytes gives for max_start_pos.  The page table must
 * cover max_start_pos + T keys.
 */
int prefill_attn_paged_dev_ex(int dtype, const void *q, int64_t q_row_stride,
                              const void *k_pool, const void *v_pool, int page_size, int num_pages,
                              const int32_t *page_table, void *out, int64_t out_row_stride,
                              int out_dtype, int T, const int32_t *start_pos_dev, int max_start_pos,
                              int num_heads, int num_kv_heads, int head_dim, int window,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * KV cache write, the step before the attention (gnosis page, "What already
 * shipped": Phase A stores each token's K/V in the cache; TensorSharp page,
 * section 4, requirement R4: global layers append at row start_pos + i,
 * sliding-window layers write slot (start_pos + i) % ring_slots).
 *   source  K of token i, kv head kh: k_src[i*src_row_stride + kh*head_dim + d]
 *           (V alike from v_src), i in 0..T-1; a fused QKV row passes
 *           k_src = row + num_heads*head_dim, v_src = k_src + num_kv_heads*head_dim
 *           and src_row_stride = (num_heads + 2*num_kv_heads)*head_dim
 *   cache   ring_slots = 0: k_cache[kh*kv_head_stride + (start_pos+i)*head_dim + d]
 *           (kv_head_stride >= (start_pos+T)*head_dim); ring_slots > 0: row
 *           (start_pos+i) % ring_slots (kv_head_stride >= ring_slots*head_dim)
 * The result is that of writing the tokens in order: in a ring shorter than
 * the chunk, only the last ring_slots tokens land.  Nothing else in the
 * cache is touched.  dtype is a PA_DTYPE_* value (the element type of source
 * and cache alike); rows of head_dim elements must be a multiple of 16
 * bytes, pointers and strides 16-byte aligned.  Sources and caches must not
 * overlap.  Asynchronous on `stream`; arguments are checked first
 * (PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED, nothing enqueued).
 */
int prefill_kv_write(int dtype, const void *k_src, const void *v_src, int64_t src_row_stride,
                     void *k_cache, void *v_cache, int64_t kv_head_stride, int ring_slots,
                     int T, int start_pos, int num_kv_heads, int head_dim, void *stream);

/*
 * Scratch bytes prefill_attn_ex (or prefill_attn_ring_ex) needs for these
 * arguments (0: none).  Returns 0 as well for arguments that are invalid or
 * unsupported.
 */
size_t prefill_attn_workspace_bytes(int dtype, int T, int start_pos, int num_heads,
                                    int num_kv_heads, int head_dim, int window);

/*
 * Launch plan for these arguments, for tests and tuning: fills up to n
 * entries of info with
 *   [0] query tokens per work-group tile     [1] query tiles
 *   [2] KV splits per tile (1: no split)     [3] work-groups launched
 *   [4] keys per KV tile                     [5] wavefronts per work-group
 *   [6] workspace bytes                      [7] KV tiles visited in total
 * and returns PA_OK or the status the same call would return.  At head_dim
 * 128 with 16-bit inputs, a causal call without a window whose query tiles
 * fill the GPU holds two query tiles per work-group (8 wavefronts, [3] =
 * ceil([1] / 2) * num_kv_heads); [7] still counts each query tile's visits.
 */
int prefill_attn_plan(int dtype, int T, int start_pos, int num_heads, int num_kv_heads,
                      int head_dim, int window, int64_t *info, int n);

/* Static text for a status code. */
const char *prefill_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PREFILL_ATTN_H */
