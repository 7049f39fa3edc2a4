/*
 * cdl.h -- C ABI of libcdl, the MI355X (gfx950) hot path of MoE token
 * dispatch and combine for one expert-parallel rank.
 *
 * The operations follow the dispatcher pages' statement of the problem:
 *   [deepep.py]   SGLang python/sglang/srt/layers/moe/token_dispatcher/deepep.py
 *   [0.4.4 diff]  sglang 0.4.4.post2 -> 0.4.4.post4 wheel diff,
 *                 sglang/srt/layers/moe/ep_moe/token_dispatcher.py
 *   [flashinfer.py] SGLang .../token_dispatcher/flashinfer.py
 *
 *   layout  (routing histogram, prefix sum, stable slot ranks)
 *     -> dispatch (row scatter: normal / low-latency padded / fp8 groups)
 *     -> [expert computation, outside this library]
 *     -> combine (gather + top-k-weighted sum per token, fp32 accumulation)
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers (hipMalloc'd or equivalent) to
 *     row-major, densely packed arrays, unless stated otherwise.  bf16 values
 *     are passed as their 16-bit patterns (uint16_t); fp8 values are OCP
 *     E4M3FN bytes (uint8_t).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on that stream and returns; nothing is
 *     synchronised and no host copy of a device value is made.
 *   - The library never allocates or frees memory and holds no global state
 *     (one exception: cdl_permute_noalloc keeps its scratch in a static device
 *     array per GPU and caches that array's address per device);
 *     the caller owns every buffer (including the layout workspace) and the
 *     "handle" that links a dispatch to its combine is the caller-owned set of
 *     arrays (src2dst, seg_indptr, counts, ll_src2dst).  Calls are
 *     thread-safe; calls that write the same buffers must be ordered by the
 *     caller (same stream or events).
 *   - Sizes: T = tokens held by this rank, H = hidden size, k = top-k
 *     (1..CDL_MAX_TOPK), L = local experts (1..CDL_MAX_LOCAL_EXPERTS),
 *     flat slot i = t*k + j.  T*k must be below 2^31.
 *   - A slot is valid for this rank iff expert_begin <= topk_ids[i] <
 *     expert_begin + L; its local expert is e_i = topk_ids[i] - expert_begin.
 *     Every other id (-1 as DeepEP marks unrouted slots, num_experts as
 *     FlashInfer's invalid id, other ranks' experts) is invalid and is
 *     dropped.
 *   - Return value: CDL_OK (0) or a negative CDL_ERR_* code.  Argument errors
 *     are detected on the host before any HIP call, so no work is enqueued.
 *     CDL_ERR_HIP means a launch failed.
 *   - Data-dependent faults (too few output rows, low-latency capacity
 *     overflow, combine map beyond the expert-output rows) never write out of
 *     bounds: the offending row is dropped and a CDL_STATUS_* bit is OR-ed into
 *     the caller's device int32 `status` word (the caller zeroes it; a NULL
 *     status pointer disables the report, not the check).
 */
#ifndef CDL_H
#define CDL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define CDL_OK 0
#define CDL_ERR_NULL_POINTER (-1)   /* a required pointer is NULL */
#define CDL_ERR_BAD_SIZE (-2)       /* negative size, k or L out of range */
#define CDL_ERR_UNSUPPORTED (-3)    /* shape the operation does not support */
#define CDL_ERR_WORKSPACE (-4)      /* workspace smaller than required */
#define CDL_ERR_TOO_LARGE (-5)      /* T*k (or a row index) needs >= 2^31 */
#define CDL_ERR_HIP (-6)            /* a kernel launch failed */
#define CDL_ERR_SCRATCH (-7)        /* cdl_permute_noalloc: more scratch than its static buffer */

/* device status bits */
#define CDL_STATUS_ROWS_OVERFLOW 1  /* a destination row >= cap_rows */
#define CDL_STATUS_LL_OVERFLOW 2    /* an expert received more than cap rows */
#define CDL_STATUS_MAP_RANGE 4      /* a combine map entry >= y_rows */
#define CDL_STATUS_REORDER_OVERFLOW 8 /* padded rows exceed the reorder_topk_ids capacity */

#define CDL_MAX_TOPK 64
#define CDL_MAX_HIDDEN (1 << 24)    /* hidden size limit of the row calls (rows are addressed
                                       with 32-bit byte offsets); larger H is CDL_ERR_TOO_LARGE */
#define CDL_MAX_LOCAL_EXPERTS 2048
#define CDL_FP8_GROUP 128

/* fp8 scale formats (bit flags) -- see cdl_dispatch_fp8_ex */
#define CDL_FP8_SCALE_UE8M0 1       /* power-of-two scales */
#define CDL_FP8_SCALE_COLMAJOR 2    /* group-major, TMA-aligned columns */
#define CDL_FP8_SCALE_PACKED 4      /* exponent bytes, 4 groups per 32-bit word (needs UE8M0) */
#define CDL_MAX_ALIGNMENT 1024
#define CDL_MAX_EXPERTS 8192        /* global experts for cdl_rank_layout */
#define CDL_MAX_RANKS 1024

/*
 * cdl_dispatch_layout_workspace_size -- bytes of device workspace that
 * cdl_dispatch_layout needs for T tokens, top-k k and L local experts
 * (per-tile expert counts).  Returns 0 for sizes the layout rejects.
 * Workspace sizing is the one-GPU counterpart of the pages' buffer size
 * hints ([deepep.py], DeepEPBuffer.get_deepep_buffer).
 */
size_t cdl_dispatch_layout_workspace_size(int64_t T, int32_t k, int32_t L);

/*
 * cdl_dispatch_layout -- the routing layout of the received tokens.
 *
 * Defined by the permute's preprocess ([0.4.4 diff],
 * _DeepEPDispatcherImplNormal._deepep_permute: deepep_run_moe_deep_preprocess
 * returns reorder_topk_ids, src2dst and seg_indptr, and the permuted buffer has
 * reorder_topk_ids.numel() rows) and the per-expert token counts of the
 * dispatch layout ([deepep.py], _DeepEPDispatcherImplNormal._dispatch_core:
 * get_dispatch_layout's num_tokens_per_expert).
 *
 *   topk_ids         in   [T, k] int32 global expert ids
 *   counts           out  [L] int32:  counts[e] = #{i : e_i = e}
 *   seg_indptr       out  [L+1] int64: exclusive prefix sum of counts;
 *                         seg_indptr[L] = R, the number of dispatched rows
 *   src2dst          out  [T*k] int32: destination row of each valid slot,
 *                         seg_indptr[e_i] + #{i' < i : e_i' = e_i} (rows of
 *                         one expert keep the flat slot order); -1 if invalid
 *   reorder_topk_ids out  [T*k] int32 capacity; the first R entries receive
 *                         the local expert of each dispatched row (so they are
 *                         nondecreasing); the rest are left untouched
 *   ws, ws_bytes          workspace of at least
 *                         cdl_dispatch_layout_workspace_size(T, k, L) bytes;
 *                         its contents need no initialisation
 * T == 0 is allowed: counts and seg_indptr are zero-filled (as the pages'
 * empty-batch path), topk_ids/src2dst/reorder may be NULL.
 * Two kernel launches: per-superblock counts, then the offsets and ranks;
 * one for small batches (T*k <= 4096, where every layout workgroup counts
 * all slots itself).
 */
int cdl_dispatch_layout(const int32_t *topk_ids, int64_t T, int32_t k,
                        int32_t expert_begin, int32_t L, int32_t *counts,
                        int64_t *seg_indptr, int32_t *src2dst,
                        int32_t *reorder_topk_ids, void *ws, size_t ws_bytes,
                        void *stream);

/*
 * cdl_dispatch_layout_aligned -- cdl_dispatch_layout with every expert
 * segment padded to a multiple of `alignment` rows ([deepep.py],
 * _DeepEPDispatcherImplNormal._dispatch_core: the normal dispatch aligns the
 * rows each local expert receives to 128 for DeepGEMM, else to 1).
 *
 *   alignment         1..CDL_MAX_ALIGNMENT
 *   counts            true (unpadded) counts
 *   seg_indptr        seg_indptr[e+1] = seg_indptr[e] + alignment*ceil(counts[e]/alignment)
 *   src2dst           seg_indptr[e_i] + rank of slot i among e_i's slots
 *   reorder_topk_ids  [reorder_cap] int32: e for the first counts[e] rows of
 *                     segment e, -1 for its padding rows; entries at or beyond
 *                     reorder_cap are not written and set
 *                     CDL_STATUS_REORDER_OVERFLOW in *status (may be NULL).
 *                     T*k + L*(alignment-1) entries always suffice.
 * Padding rows of the dispatched buffer are never written by any dispatch.
 * Rejects T*k + L*(alignment-1) >= 2^31 with CDL_ERR_TOO_LARGE.
 */
int cdl_dispatch_layout_aligned(const int32_t *topk_ids, int64_t T, int32_t k,
                                int32_t expert_begin, int32_t L, int32_t alignment,
                                int32_t *counts, int64_t *seg_indptr, int32_t *src2dst,
                                int32_t *reorder_topk_ids, int64_t reorder_cap, int32_t *status,
                                void *ws, size_t ws_bytes, void *stream);

/*
 * cdl_permute -- layout and normal-mode scatter in one call, the older
 * dispatcher's permute step ([0.4.4 diff],
 * _DeepEPDispatcherImplNormal._deepep_permute: preprocess the received top-k
 * ids into reorder_topk_ids / src2dst / seg_indptr, then copy every token row
 * to its destination rows).  Two kernel launches (one for small batches,
 * T*k <= 4096); the row loads are issued before the layout arithmetic.
 *
 * Layout arguments and outputs are exactly those of
 * cdl_dispatch_layout_aligned (alignment 1 gives cdl_dispatch_layout's; same
 * workspace size); x, out, cap_rows and status as for cdl_dispatch.
 * R (the padded row count seg_indptr[L]) is not known before the call: `out`
 * must hold cap_rows rows with cap_rows an upper bound (T*k + L*(alignment-1)
 * always suffices) or a known R; a destination at or beyond cap_rows is
 * dropped and sets CDL_STATUS_ROWS_OVERFLOW.  Padding rows are not written.
 * Requires H % 8 == 0 and 16-byte aligned x and out (CDL_ERR_UNSUPPORTED
 * otherwise).
 */
int cdl_permute(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                int32_t expert_begin, int32_t L, int32_t alignment, int32_t *counts,
                int64_t *seg_indptr, int32_t *src2dst, int32_t *reorder_topk_ids,
                int64_t reorder_cap, uint16_t *out, int64_t cap_rows, int32_t *status, void *ws,
                size_t ws_bytes, void *stream);

/*
 * cdl_permute_noalloc -- cdl_permute for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, outputs and errors as cdl_permute, without the
 * workspace: the layout's scratch (the superblock counts) lives in a static
 * device array of CDL_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends.  Its device address is looked up once per
 * device (hipGetSymbolAddress, with that device current) on the first call
 * there; no call allocates or frees memory.  Calls whose
 * cdl_dispatch_layout_workspace_size(T, k, L) exceeds the buffer return
 * CDL_ERR_SCRATCH before any work (realistic shapes fit: 4096 tokens of
 * top-8 over 32 experts need 4.3 KB).  `stream` must belong to the current
 * device (CDL_ERR_UNSUPPORTED otherwise).  The buffer needs no clearing
 * between calls; it keeps the last call's contents.  Calls that overlap on
 * one GPU (other streams, other host threads) share that GPU's buffer and
 * race: order them (one stream, or events).
 */
#define CDL_NOALLOC_SCRATCH_BYTES (1 << 20)
int cdl_permute_noalloc(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                        const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                        int32_t alignment, int32_t *counts, int64_t *seg_indptr, int32_t *src2dst,
                        int32_t *reorder_topk_ids, int64_t reorder_cap, uint16_t *out,
                        int64_t cap_rows, int32_t *status, void *stream);

/*
 * cdl_permute_fp8 -- cdl_permute with the per-token, per-128-group fp8
 * quantisation of cdl_dispatch_fp8_ex on the scatter ([deepep.py],
 * _DeepEPDispatcherImplNormal.dispatch_a).  out_q [cap_rows, H] E4M3FN bytes;
 * out_scales in the scale_flags format for cap_rows rows (one column-major
 * matrix of cap_rows rows).  Requires H % 128 == 0, 16-byte aligned x,
 * 8-byte aligned out_q and 4-byte aligned out_scales.
 */
int cdl_permute_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                    int32_t expert_begin, int32_t L, int32_t alignment, int32_t *counts,
                    int64_t *seg_indptr, int32_t *src2dst, int32_t *reorder_topk_ids,
                    int64_t reorder_cap, uint8_t *out_q, void *out_scales, int32_t scale_flags,
                    int64_t cap_rows, int32_t *status, void *ws, size_t ws_bytes, void *stream);

/*
 * cdl_permute_fp8_tensor -- cdl_permute with the permuted rows cast to fp8
 * per tensor: the older permute allocates its buffer in the fp8 dtype for
 * per-tensor w8a8 weights (not block-quantised) and passes its permute kernel
 * no input scale ([0.4.4 diff], _DeepEPDispatcherImplNormal._deepep_permute:
 * gateup_input's dtype).  Every element of a dispatched row becomes
 *     e4m3fn_rne(clamp(fl32(x / s), -448, 448)),
 * s the per-tensor scale, with no per-row scales written.
 *
 *   out_q  out [cap_rows, H] E4M3FN bytes (8-byte aligned); rows at or beyond
 *          cap_rows are dropped with CDL_STATUS_ROWS_OVERFLOW, padding rows
 *          are not written
 *   scale  in  device pointer to one fp32 s > 0 (finite), or NULL for s = 1
 *          (the pages' None); a power of two is applied exactly through its
 *          inverse, any other value by a correctly rounded division
 * Layout arguments, workspace, x, cap_rows and status as for cdl_permute.
 * Requires H % 8 == 0 and 16-byte aligned x (CDL_ERR_UNSUPPORTED otherwise).
 */
int cdl_permute_fp8_tensor(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                           const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                           int32_t alignment, int32_t *counts, int64_t *seg_indptr,
                           int32_t *src2dst, int32_t *reorder_topk_ids, int64_t reorder_cap,
                           uint8_t *out_q, const float *scale, int64_t cap_rows, int32_t *status,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * cdl_permute_fp8_workspace_size -- workspace bytes for cdl_permute_fp8
 * (rows = cap_rows) and cdl_permute_ll_fp8 (rows = L * cap) in the given
 * scale format: cdl_dispatch_layout_workspace_size(T, k, L) for every valid
 * format (column-major scales are written in place, each scale word with the
 * temporal cache policy so that the L2 merges the words a line receives from
 * 32 rows before they reach memory).  0 for invalid arguments (H not a
 * multiple of 128, bad flags).
 */
size_t cdl_permute_fp8_workspace_size(int64_t T, int32_t k, int32_t L, int64_t H,
                                      int32_t scale_flags, int64_t rows);

/*
 * cdl_rank_layout_workspace_size -- device workspace bytes for
 * cdl_rank_layout (0 for rejected sizes).
 */
size_t cdl_rank_layout_workspace_size(int64_t T, int32_t k, int32_t E, int32_t num_ranks,
                                      int32_t ranks_per_node);

/*
 * cdl_rank_layout -- where a token batch goes before the exchange
 * ([deepep.py], _DeepEPDispatcherImplNormal._dispatch_core:
 * get_dispatch_layout returns num_tokens_per_rank, num_tokens_per_rdma_rank,
 * num_tokens_per_expert and is_token_in_rank).
 *
 *   topk_ids                  in  [T, k] int32 global ids; an id outside [0, E)
 *                                 is an unrouted slot
 *   E, num_ranks              E % num_ranks == 0; rank r owns experts
 *                             [r*E/num_ranks, (r+1)*E/num_ranks)
 *   ranks_per_node            num_ranks % ranks_per_node == 0 (node = RDMA rank)
 *   num_tokens_per_rank       out [num_ranks] int32: tokens with >= 1 slot on r
 *   num_tokens_per_rdma_rank  out [num_ranks/ranks_per_node] int32: tokens with
 *                             >= 1 slot on the node's ranks (may be NULL)
 *   num_tokens_per_expert     out [E] int32: slots per expert
 *   is_token_in_rank          out [T, num_ranks] bytes, 1 if token t has a slot
 *                             on rank r, else 0 (torch.bool compatible)
 *   ws, ws_bytes              cdl_rank_layout_workspace_size bytes, no
 *                             initialisation needed
 * CDL_ERR_UNSUPPORTED for indivisible sizes; E <= CDL_MAX_EXPERTS and
 * num_ranks <= CDL_MAX_RANKS.  Two kernel launches, no atomics outside
 * workgroups (the counts are deterministic).
 */
int cdl_rank_layout(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E, int32_t num_ranks,
                    int32_t ranks_per_node, int32_t *num_tokens_per_rank,
                    int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                    uint8_t *is_token_in_rank, void *ws, size_t ws_bytes, void *stream);

/*
 * cdl_dispatch -- normal-mode bf16 row scatter ([0.4.4 diff],
 * _deepep_permute: the PreReorder permute copies every token row to the
 * destination rows src2dst names; it takes no weights).
 *
 *   x        in   [T, H] bf16 token rows
 *   src2dst  in   [T*k] int32 from cdl_dispatch_layout
 *   out      out  [cap_rows, H] bf16; out[src2dst[t*k+j], :] = x[t, :] bit for
 *                 bit for every valid slot; no other row is written
 *   cap_rows      rows allocated in `out` (normally R); a destination at or
 *                 beyond it is dropped and sets CDL_STATUS_ROWS_OVERFLOW
 *   status   out  device int32 status word (may be NULL)
 * Any H >= 1 is accepted (H % 8 == 0 with 16-byte aligned rows takes the
 * vector path).
 */
int cdl_dispatch(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                 const int32_t *src2dst, uint16_t *out, int64_t cap_rows,
                 int32_t *status, void *stream);

/*
 * cdl_dispatch_fp8 -- normal-mode scatter with per-token, per-group fp8
 * quantisation on the way ([deepep.py], _DeepEPDispatcherImplNormal.dispatch_a:
 * the per-token group quant with a hard-coded group of 128 before a normal
 * fp8 dispatch; scales row-major fp32).
 *
 * For every token row with at least one valid slot and every group g of
 * CDL_FP8_GROUP contiguous elements: a = max |x|, s = a / 448 (IEEE binary32
 * division), q = e4m3fn_rne(clamp(x / s, -448, 448)) (a = 0 gives s = 0 and
 * the signed zero of each element).  The (q, s) row is written to every
 * destination row.
 *
 *   out_q       out  [cap_rows, H] E4M3FN bytes
 *   out_scales  out  [cap_rows, H / 128] fp32
 * Requires H % 128 == 0 (CDL_ERR_UNSUPPORTED otherwise) and 16-byte aligned
 * rows.
 */
int cdl_dispatch_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                     const int32_t *src2dst, uint8_t *out_q, float *out_scales,
                     int64_t cap_rows, int32_t *status, void *stream);

/*
 * cdl_fp8_scale_bytes -- bytes of a scale buffer for `rows` destination rows
 * of H elements in the scale_flags format; for column-major formats every
 * rows_per_mat rows form one matrix (normal dispatch: rows_per_mat = rows =
 * cap_rows; low latency: rows = L*cap, rows_per_mat = cap).  0 for invalid
 * arguments.
 */
size_t cdl_fp8_scale_bytes(int64_t rows, int64_t H, int32_t scale_flags, int64_t rows_per_mat);

/*
 * cdl_dispatch_fp8_ex -- cdl_dispatch_fp8 with a choice of scale format, the
 * switches of the group quant that feeds DeepGEMM ([deepep.py],
 * _DeepEPDispatcherImplNormal.dispatch_a: column_major_scales,
 * scale_tma_aligned, scale_ue8m0; _DeepEPDispatcherImplLowLatency.
 * _dispatch_core: round_scale / use_ue8m0 give int32-packed UE8M0 scales).
 * scale_flags, a combination of:
 *   0                        fp32 scales s = amax / 448, row-major [rows][G]
 *                            (exactly cdl_dispatch_fp8)
 *   CDL_FP8_SCALE_UE8M0      the scale is the smallest power of two p >=
 *                            2^-127 with 448 * p >= amax; q = e4m3(x / p) is
 *                            an exact scaling (no clamp); a zero group gets
 *                            p = 2^-127
 *   CDL_FP8_SCALE_COLMAJOR   scales stored group-major, [G][ld] fp32 with
 *                            ld = cap_rows rounded up to a multiple of 4 (every
 *                            column 16-byte aligned); rows [cap_rows, ld) of
 *                            each column are never written
 *   CDL_FP8_SCALE_PACKED     (requires UE8M0) the exponent byte log2(p) + 127,
 *                            four consecutive groups per 32-bit word, group g
 *                            in byte g % 4; row-major [rows][ceil(G/4)] words
 *                            or, with COLMAJOR, [ceil(G/4)][ld] words
 * out_scales must hold cdl_fp8_scale_bytes(cap_rows, H, scale_flags,
 * cap_rows) bytes.  CDL_ERR_UNSUPPORTED for an invalid combination.
 */
int cdl_dispatch_fp8_ex(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                        const int32_t *src2dst, uint8_t *out_q, void *out_scales,
                        int32_t scale_flags, int64_t cap_rows, int32_t *status, void *stream);

/*
 * cdl_dispatch_ll -- low-latency dispatch into a padded per-expert buffer
 * ([deepep.py], _DeepEPDispatcherImplLowLatency._dispatch_core:
 * low_latency_dispatch returns the packed receive buffer and its per-expert
 * counts, which DeepEPLLDispatchOutput carries as masked_m).
 *
 *   topk_ids, expert_begin, L   as for cdl_dispatch_layout
 *   src2dst, seg_indptr, counts from cdl_dispatch_layout on the same ids
 *   cap         rows per expert in `out`
 *   out         out [L, cap, H] bf16; the slot of valid (t, j) in expert e_i's
 *               block is src2dst[i] - seg_indptr[e_i] (ascending token order);
 *               rows at or beyond masked_m[e] are never written
 *   masked_m    out [L] int32: min(counts[e], cap)
 *   ll_src2dst  out [T*k] int32: e_i*cap + slot, or -1 (invalid or dropped)
 *   status      out device int32 (may be NULL): CDL_STATUS_LL_OVERFLOW when an
 *               expert has more than cap rows (the extra rows are dropped)
 */
int cdl_dispatch_ll(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                    const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                    const int32_t *src2dst, const int64_t *seg_indptr,
                    const int32_t *counts, int64_t cap, uint16_t *out,
                    int32_t *masked_m, int32_t *ll_src2dst, int32_t *status,
                    void *stream);

/*
 * cdl_permute_ll -- the low-latency dispatch in one call: the routing layout
 * and the scatter into the padded per-expert buffer ([deepep.py],
 * _DeepEPDispatcherImplLowLatency._dispatch_core: one low_latency_dispatch
 * call returns the packed receive buffer and the per-expert counts).
 *
 * Outputs are exactly those of cdl_dispatch_layout (counts, seg_indptr,
 * src2dst, and reorder_topk_ids if reorder_cap > 0; it may be NULL with
 * reorder_cap 0) followed by cdl_dispatch_ll on them (out [L, cap, H] bf16,
 * masked_m, ll_src2dst, CDL_STATUS_LL_OVERFLOW); ws as for
 * cdl_dispatch_layout.  One kernel launch for small batches (T*k <= 4096,
 * e.g. 128 tokens of top-8), two otherwise.  Requires H % 8 == 0 and 16-byte aligned x and out.
 */
int cdl_permute_ll(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                   int32_t expert_begin, int32_t L, int32_t *counts, int64_t *seg_indptr,
                   int32_t *src2dst, int32_t *reorder_topk_ids, int64_t reorder_cap, int64_t cap,
                   uint16_t *out, int32_t *masked_m, int32_t *ll_src2dst, int32_t *status, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * cdl_permute_ll_fp8 -- cdl_permute_ll with the fp8 rows and scales of
 * cdl_dispatch_ll_fp8 (out_q [L, cap, H] E4M3FN bytes; out_scales in the
 * scale_flags format for L*cap rows, every expert's cap rows one
 * column-major matrix).  Requires H % 128 == 0.
 */
int cdl_permute_ll_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                       const int32_t *topk_ids, int32_t expert_begin, int32_t L, int32_t *counts,
                       int64_t *seg_indptr, int32_t *src2dst, int32_t *reorder_topk_ids,
                       int64_t reorder_cap, int64_t cap, uint8_t *out_q, void *out_scales,
                       int32_t scale_flags, int32_t *masked_m, int32_t *ll_src2dst,
                       int32_t *status, void *ws, size_t ws_bytes, void *stream);

/*
 * cdl_dispatch_ll_fp8 -- cdl_dispatch_ll with fp8 rows ([deepep.py],
 * _DeepEPDispatcherImplLowLatency._dispatch_core: low_latency_dispatch with
 * use_fp8 returns the packed rows with their scales).  out_q [L, cap, H]
 * E4M3FN bytes; out_scales in the scale_flags format of cdl_dispatch_fp8_ex
 * for L*cap rows where every expert's cap rows form one column-major matrix
 * (rows_per_mat = cap).  Slots, masked_m, ll_src2dst and overflow handling
 * are those of cdl_dispatch_ll.
 */
int cdl_dispatch_ll_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                        const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                        const int32_t *src2dst, const int64_t *seg_indptr, const int32_t *counts,
                        int64_t cap, uint8_t *out_q, void *out_scales, int32_t scale_flags,
                        int32_t *masked_m, int32_t *ll_src2dst, int32_t *status, void *stream);

/*
 * cdl_combine -- gather the expert outputs back and form each token's
 * top-k-weighted sum ([0.4.4 diff], _DeepEPDispatcherImplNormal.combine_a: the
 * post-reorder takes the expert outputs, src2dst, topk_ids and topk_weights and
 * writes [T, H] in the input dtype; [deepep.py],
 * _DeepEPDispatcherImplLowLatency._combine_core: low_latency_combine takes the
 * weights too).
 *
 *   y             in  [y_rows, H] bf16 expert outputs (the normal buffer, or
 *                     the low-latency buffer viewed as [L*cap, H])
 *   map           in  [T*k] int32: src2dst (normal) or ll_src2dst (low latency)
 *   topk_weights  in  [T, k] fp32
 *   out           out [T, H] bf16:
 *                     out[t, h] = bf16_rne(fma chain over valid j ascending of
 *                     w[t, j] * y[map[t*k+j], h], from +0 in fp32);
 *                     a token with no valid slot gets +0
 *   status        out device int32 (may be NULL): CDL_STATUS_MAP_RANGE for a
 *                     map entry >= y_rows (that slot is skipped)
 * `out` must not overlap `y`.
 */
int cdl_combine(const uint16_t *y, int64_t y_rows, int64_t H, const int32_t *map,
                const float *topk_weights, int64_t T, int32_t k, uint16_t *out,
                int32_t *status, void *stream);

/*
 * cdl_combine_timed -- cdl_combine whose kernel launch carries two events
 * for measurement: start_event and stop_event (hipEvent_t created with
 * timing enabled, either may be NULL) receive the begin and end of the
 * combine kernel itself, so hipEventElapsedTime between them is the
 * kernel's duration, without the extra queue packets (and the dependency
 * round trips) that a separate event record adds between kernels.  Results
 * and errors are those of cdl_combine.
 */
int cdl_combine_timed(const uint16_t *y, int64_t y_rows, int64_t H, const int32_t *map,
                      const float *topk_weights, int64_t T, int32_t k, uint16_t *out,
                      int32_t *status, void *start_event, void *stop_event, void *stream);

/*
 * cdl_ll_expected_m -- host-side hint for the masked grouped GEMM after a
 * low-latency dispatch ([deepep.py], _DeepEPDispatcherImplLowLatency.dispatch_a):
 * (T * num_ranks * k + E) / E with integer division.  Returns -1 for E <= 0 or
 * negative sizes.  Pure host function.
 */
int64_t cdl_ll_expected_m(int64_t T, int32_t num_ranks, int32_t k, int32_t E);

/*
 * cdl_status_string -- static text for a CDL_OK / CDL_ERR_* return code.
 *
 * The return codes stand in for the exceptions the dispatcher pages raise
 * before any dispatch work starts: [deepep.py] _DeepEPDispatcherImplBase.__init__
 * raises ImportError when the communication library is missing (here: the
 * HIP library is loaded or the binding refuses, and CDL_ERR_HIP reports a
 * failed launch); _DeepEPDispatcherImplBase._validate_and_adjust_dtype raises
 * RuntimeError for an output dtype the hardware cannot produce and
 * _DeepEPDispatcherImplNormal.combine_a raises NotImplementedError for a
 * runner that is not supported (here: CDL_ERR_UNSUPPORTED for a shape,
 * alignment or scale format the operation does not support);
 * DeepEPDispatcher._get_impl raises ValueError for an invalid mode (here:
 * CDL_ERR_BAD_SIZE / CDL_ERR_TOO_LARGE / CDL_ERR_NULL_POINTER /
 * CDL_ERR_WORKSPACE for invalid arguments).  Unlike the exceptions, every
 * code is returned on the host before any work is enqueued (CDL_ERR_HIP
 * aside), so a failed call leaves every output untouched.
 *
 * Returns a pointer to a static NUL-terminated string owned by the library
 * (never NULL; "unknown cdl status code" for a value that is not a code).
 * Pure host function, thread-safe.
 */
const char *cdl_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* CDL_H */
