/*
 * cdl_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, single-threaded CPU oracle for the single-GPU hot path of
 * MoE token dispatch and combine (one expert-parallel rank's share).  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code, header, table or helper with the HIP
 * library; both sides only receive the same seeded inputs.
 *
 * Every function below states the passage of the pages it follows.  Page
 * names used in the citations:
 *   [deepep.py]  SGLang python/sglang/srt/layers/moe/token_dispatcher/deepep.py
 *                (main branch): the current DeepEP dispatcher.
 *   [0.4.4 diff] sglang 0.4.4.post2 -> 0.4.4.post4 wheel diff of
 *                sglang/srt/layers/moe/ep_moe/token_dispatcher.py: the older
 *                DeepEP dispatcher with the rank-local permute / post-reorder.
 *   [flashinfer.py] SGLang .../token_dispatcher/flashinfer.py (main branch).
 *
 * Arithmetic conventions (readings of the pages where they are silent):
 *   - bf16 values are passed as their 16-bit patterns (uint16_t), fp8-e4m3fn
 *     values as bytes.  Decoding and RNE encoding are written below from the
 *     format definitions (IEEE-754 binary32 truncated to its upper half for
 *     bf16; OCP 8-bit floating point E4M3 "fn": bias 7, no infinities, one
 *     NaN mantissa pattern, max finite 448).
 *   - The combine accumulates in binary32 with a correctly rounded fused
 *     multiply-add per valid slot in ascending slot order from +0, then
 *     rounds once to bf16 (fp32 accumulation is fixed by the hot path's
 *     statement of the problem).  oracle_combine_f64 gives the fp64 value of
 *     the same sum, to pin the fp32 result within one bf16 ulp.
 *   - The fp8 group quantisation works in binary32 (the scales are fp32):
 *     a = max|x|, s = a / 448, q = e4m3(clamp(x / s, -448, 448)), each
 *     division correctly rounded; an all-zero group gets s = 0 and the signed
 *     zero of each element.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off -fno-fast-math
 *        (contraction off, so that only the explicit fmaf() fuses).
 *
 * Parity pins (tests that check this file against something other than
 * itself) live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats, from their definitions.                                   */
/* ------------------------------------------------------------------------ */

/* Round a non-negative double holding an exact multiple count (a / quantum,
 * computed exactly) to the nearest integer, ties to even. */
static double round_half_even(double q)
{
    double fl = floor(q);
    double d = q - fl;
    if (d > 0.5)
        return fl + 1.0;
    if (d < 0.5)
        return fl;
    return (fmod(fl, 2.0) != 0.0) ? fl + 1.0 : fl;
}

static uint32_t f32_bits(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    return u;
}

static float f32_from_bits(uint32_t u)
{
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

/* bf16 -> fp32: a bf16 pattern is the upper half of the binary32 pattern of
 * the same value, so the value is that pattern followed by 16 zero bits. */
float oracle_bf16_to_f32(uint16_t b)
{
    return f32_from_bits((uint32_t)b << 16);
}

/* fp32 -> bf16, round to nearest, ties to even.  The value is first rounded
 * onto the bf16 grid (8 significant bits; below 2^-126 the grid step is fixed
 * at 2^-133, the bf16 subnormal step), then encoded: a value on the bf16 grid
 * is a binary32 value whose lower 16 pattern bits are zero. */
uint16_t oracle_bf16_rne(float v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v) || v == 0.0f)
        return (uint16_t)(f32_bits(v) >> 16);
    double a = fabs((double)v);
    int ex;
    (void)frexp(a, &ex);            /* a = f * 2^ex with f in [0.5, 1) */
    int e = ex - 1;                 /* a in [2^e, 2^(e+1)) */
    if (e < -126)
        e = -126;
    double quantum = ldexp(1.0, e - 7);
    double r = round_half_even(a / quantum) * quantum;
    if (r >= ldexp(1.0, 128))       /* rounds past the largest finite bf16 */
        return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r;            /* exact: r lies on the bf16 grid */
    return (uint16_t)(sign | (f32_bits(rf) >> 16));
}

/* e4m3fn -> fp32 (OCP FP8 E4M3: bias 7; exponent field 0 is subnormal with
 * step 2^-9; the all-ones pattern S.1111.111 is NaN; there is no infinity). */
float oracle_e4m3fn_to_f32(uint8_t b)
{
    int s = (b >> 7) & 1;
    int E = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (E == 15 && m == 7)
        return s ? -NAN : NAN;
    if (E == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, E - 7);
    return (float)(s ? -v : v);
}

/* fp32 -> e4m3fn, round to nearest, ties to even, sign kept on zero.
 * Domain: |v| <= 448 (the method clamps before converting); outside it, and
 * for NaN, the NaN pattern is returned. */
uint8_t oracle_e4m3fn_rne(float v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    if (isnan(v))
        return (uint8_t)(sign | 0x7Fu);
    double a = fabs((double)v);
    if (a > 448.0)
        return (uint8_t)(sign | 0x7Fu);
    if (a == 0.0)
        return sign;
    int ex;
    (void)frexp(a, &ex);
    int e = ex - 1;                 /* a in [2^e, 2^(e+1)) */
    if (e < -6)
        e = -6;                     /* subnormal range: step 2^-9 */
    double q = round_half_even(a / ldexp(1.0, e - 3));   /* 0 .. 16 */
    if (q >= 16.0) {                /* rounded up to the next binade */
        e += 1;
        q = 8.0;
    }
    if (q < 8.0)                    /* only reachable when e == -6 */
        return (uint8_t)(sign | (uint8_t)q);
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8)));
}

/* The e4m3fn NaN pattern S.1111.111 carrying the sign of the bf16 value x. */
static uint8_t nan_code_of(uint16_t x) { return (uint8_t)(((x >> 8) & 0x80u) | 0x7Fu); }

/* ------------------------------------------------------------------------ */
/* Routing layout.                                                           */
/* ------------------------------------------------------------------------ */

/* Local expert of a top-k slot: id - expert_begin when the id lies in
 * [expert_begin, expert_begin + L), else -1.  Covers every invalid encoding
 * on the pages: -1 for unrouted DeepEP slots ([deepep.py], the AITER sink-slot
 * comment in DeepEPDispatcher.__init__), num_experts as FlashInfer's invalid
 * expert id ([flashinfer.py], FlashinferDispatcher.__init__) and the experts
 * of other ranks. */
static int32_t local_expert(int32_t id, int32_t expert_begin, int32_t L)
{
    int64_t e = (int64_t)id - (int64_t)expert_begin;
    return (e >= 0 && e < (int64_t)L) ? (int32_t)e : -1;
}

/* The layout the permute consumes ([0.4.4 diff],
 * _DeepEPDispatcherImplNormal._deepep_permute: deepep_run_moe_deep_preprocess
 * returns reorder_topk_ids, src2dst and seg_indptr; the permuted buffer has
 * reorder_topk_ids.numel() rows; seg_indptr is int64 and all zero for an
 * empty batch) plus the per-expert counts ([deepep.py], _dispatch_core:
 * num_tokens_per_expert / num_recv_tokens_per_expert).
 *
 * A stable counting sort of the flat slots i = t*k + j by local expert:
 *   counts[e]       = #{i : e_i = e}
 *   seg_indptr[0]   = 0, seg_indptr[e+1] = seg_indptr[e] + counts[e]
 *   src2dst[i]      = seg_indptr[e_i] + #{i' < i : e_i' = e_i}, or -1
 *   reorder[src2dst[i]] = e_i
 * Returns R = seg_indptr[L], the number of dispatched rows. */
int64_t oracle_layout(const int32_t *topk_ids, int64_t T, int32_t k,
                      int32_t expert_begin, int32_t L, int32_t *counts,
                      int64_t *seg_indptr, int32_t *src2dst,
                      int32_t *reorder_topk_ids)
{
    int64_t n = T * (int64_t)k;
    for (int32_t e = 0; e < L; ++e)
        counts[e] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = local_expert(topk_ids[i], expert_begin, L);
        if (e >= 0)
            counts[e] += 1;
    }
    seg_indptr[0] = 0;
    for (int32_t e = 0; e < L; ++e)
        seg_indptr[e + 1] = seg_indptr[e] + counts[e];

    int64_t *cursor = (int64_t *)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
    if (!cursor)
        return -1;
    for (int32_t e = 0; e < L; ++e)
        cursor[e] = seg_indptr[e];
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = local_expert(topk_ids[i], expert_begin, L);
        if (e < 0) {
            src2dst[i] = -1;
            continue;
        }
        int64_t d = cursor[e]++;
        src2dst[i] = (int32_t)d;
        reorder_topk_ids[d] = e;
    }
    free(cursor);
    return seg_indptr[L];
}

/* Layout with every expert segment padded to a multiple of `alignment` rows
 * ([deepep.py], _DeepEPDispatcherImplNormal._dispatch_core: the normal
 * dispatch aligns the rows each local expert receives to 128 when the
 * grouped GEMM is DeepGEMM, else to 1).  Reading: counts stay the true
 * counts; seg_indptr[e+1] = seg_indptr[e] + alignment * ceil(counts[e] /
 * alignment); real rows keep the stable order at the start of their segment;
 * padding rows belong to no slot and their reorder_topk_ids entry is -1.
 * reorder_topk_ids must hold seg_indptr[L] entries.  Returns seg_indptr[L]. */
int64_t oracle_layout_aligned(const int32_t *topk_ids, int64_t T, int32_t k,
                              int32_t expert_begin, int32_t L, int32_t alignment,
                              int32_t *counts, int64_t *seg_indptr, int32_t *src2dst,
                              int32_t *reorder_topk_ids)
{
    if (alignment < 1)
        return -1;
    int64_t n = T * (int64_t)k;
    for (int32_t e = 0; e < L; ++e)
        counts[e] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = local_expert(topk_ids[i], expert_begin, L);
        if (e >= 0)
            counts[e] += 1;
    }
    seg_indptr[0] = 0;
    for (int32_t e = 0; e < L; ++e) {
        int64_t padded = ((int64_t)counts[e] + alignment - 1) / alignment * alignment;
        seg_indptr[e + 1] = seg_indptr[e] + padded;
    }
    for (int32_t e = 0; e < L; ++e)
        for (int64_t r = seg_indptr[e]; r < seg_indptr[e + 1]; ++r)
            reorder_topk_ids[r] = (r < seg_indptr[e] + counts[e]) ? e : -1;
    int64_t *cursor = (int64_t *)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
    if (!cursor)
        return -1;
    for (int32_t e = 0; e < L; ++e)
        cursor[e] = seg_indptr[e];
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = local_expert(topk_ids[i], expert_begin, L);
        src2dst[i] = e < 0 ? -1 : (int32_t)cursor[e]++;
    }
    free(cursor);
    return seg_indptr[L];
}

/* Rank layout of a token batch before the exchange ([deepep.py],
 * _DeepEPDispatcherImplNormal._dispatch_core: get_dispatch_layout(topk_ids,
 * num_experts) returns num_tokens_per_rank, num_tokens_per_rdma_rank,
 * num_tokens_per_expert and is_token_in_rank).  Ids are global; an id outside
 * [0, E) marks an unrouted slot.  Rank r owns experts [r*E/R, (r+1)*E/R);
 * node n owns ranks [n*rpn, (n+1)*rpn).
 *   per_expert[e]   = number of slots with id e
 *   in_rank[t*R+r]  = 1 if token t has a slot on rank r, else 0
 *   per_rank[r]     = number of tokens with in_rank[t][r] = 1
 *   per_node[n]     = number of tokens with a slot on any rank of node n
 * Returns -1 if E is not a multiple of R or R of rpn. */
int32_t oracle_rank_layout(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                           int32_t R, int32_t rpn, int32_t *per_rank, int32_t *per_node,
                           int32_t *per_expert, uint8_t *in_rank)
{
    if (E <= 0 || R <= 0 || rpn <= 0 || E % R != 0 || R % rpn != 0)
        return -1;
    int32_t epr = E / R;
    int32_t N = R / rpn;
    for (int32_t r = 0; r < R; ++r)
        per_rank[r] = 0;
    for (int32_t n = 0; n < N; ++n)
        per_node[n] = 0;
    for (int32_t e = 0; e < E; ++e)
        per_expert[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        uint8_t *row = in_rank + t * R;
        for (int32_t r = 0; r < R; ++r)
            row[r] = 0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t id = topk_ids[t * k + j];
            if (id < 0 || id >= E)
                continue;
            per_expert[id] += 1;
            row[id / epr] = 1;
        }
        for (int32_t r = 0; r < R; ++r)
            per_rank[r] += row[r];
        for (int32_t n = 0; n < N; ++n) {
            int any = 0;
            for (int32_t r = n * rpn; r < (n + 1) * rpn; ++r)
                any |= row[r];
            per_node[n] += any;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch.                                                                 */
/* ------------------------------------------------------------------------ */

/* Normal-mode row scatter ([0.4.4 diff], _deepep_permute: the PreReorder
 * permute copies each token row to the destination rows src2dst names; it is
 * given no weights).  P[src2dst[t*k+j], :] = x[t, :] bit for bit for every
 * valid slot.  Rows of P that no slot names are left untouched. */
void oracle_dispatch(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                     const int32_t *src2dst, uint16_t *P)
{
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int32_t d = src2dst[t * k + j];
            if (d >= 0)
                memcpy(P + (int64_t)d * H, x + t * H, sizeof(uint16_t) * (size_t)H);
        }
}

/* Low-latency dispatch into a padded [L, cap, H] buffer ([deepep.py],
 * _DeepEPDispatcherImplLowLatency._dispatch_core: low_latency_dispatch returns
 * the packed receive buffer and packed_recv_count, which becomes masked_m of
 * DeepEPLLDispatchOutput).  The slot of a valid (t, j) inside its expert's
 * block is its rank among the slots of that expert in ascending flat order
 * (computed here directly, not from the normal layout).  A slot whose rank
 * reaches cap is dropped, its ll_src2dst entry is -1 and the return value is
 * nonzero (the pages fail such a case with an assert or an illegal access;
 * the reading here is drop-and-flag).  masked_m[e] = min(count_e, cap).
 * Padding rows are never written. */
int32_t oracle_dispatch_ll(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                           const int32_t *topk_ids, int32_t expert_begin,
                           int32_t L, int64_t cap, uint16_t *B,
                           int32_t *masked_m, int32_t *ll_src2dst)
{
    int32_t overflow = 0;
    int64_t *seen = (int64_t *)calloc((size_t)(L > 0 ? L : 1), sizeof(int64_t));
    if (!seen)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t i = t * k + j;
            int32_t e = local_expert(topk_ids[i], expert_begin, L);
            if (e < 0) {
                ll_src2dst[i] = -1;
                continue;
            }
            int64_t slot = seen[e]++;
            if (slot >= cap) {
                ll_src2dst[i] = -1;
                overflow = 1;
                continue;
            }
            int64_t row = (int64_t)e * cap + slot;
            memcpy(B + row * H, x + t * H, sizeof(uint16_t) * (size_t)H);
            ll_src2dst[i] = (int32_t)row;
        }
    for (int32_t e = 0; e < L; ++e)
        masked_m[e] = (int32_t)(seen[e] < cap ? seen[e] : cap);
    free(seen);
    return overflow;
}

/* Per-tensor fp8 cast of n bf16 values: the permuted buffer of the older
 * permute is fp8 when the weights are w8a8 per tensor ([0.4.4 diff],
 * _DeepEPDispatcherImplNormal._deepep_permute: gateup_input is allocated in
 * the fp8 dtype unless the quantisation is block-wise, and the permute kernel
 * receives no scale, None, in the place of an input scale).  Reading: the
 * per-tensor scale s divides every element (s = 1 when none is given), the
 * quotient is clamped to [-448, 448] (saturation to the largest finite
 * e4m3fn) and rounded to e4m3fn, ties to even:
 *   q = e4m3fn_rne(clamp(fl(x / s), -448, 448)),  s > 0 finite.
 * Non-finite x (the pages are silent): +-inf saturates to +-448 like any
 * other quotient beyond the range, and a NaN quotient becomes the e4m3fn NaN
 * code with the sign of x (stated explicitly: the sign of a NaN produced by
 * arithmetic is left open by IEEE 754). */
void oracle_cast_fp8_tensor(const uint16_t *x, int64_t n, float s, uint8_t *q)
{
    for (int64_t c = 0; c < n; ++c) {
        float v = oracle_bf16_to_f32(x[c]) / s;
        if (v > 448.0f)
            v = 448.0f;
        if (v < -448.0f)
            v = -448.0f;
        q[c] = isnan(v) ? nan_code_of(x[c]) : oracle_e4m3fn_rne(v);
    }
}

/* Per-token, per-group fp8 quantisation of one group of n bf16 values
 * ([deepep.py], _DeepEPDispatcherImplNormal.dispatch_a: per-token group quant
 * with a hard-coded group of 128 before a normal fp8 dispatch).  Reading of
 * the scale: s = amax / 448 (448 = largest finite e4m3fn), the elements are
 * divided by s, clamped to [-448, 448] and rounded to e4m3fn, ties to even.
 * Non-finite elements (the pages are silent): NaN elements do not enter
 * amax (an infinity does, and then s = inf, so finite elements quantise to
 * signed zeros); a NaN quotient (a NaN x, or inf / inf) becomes the e4m3fn
 * NaN code with the sign of x. */
void oracle_quant_group_fp8(const uint16_t *x, int64_t n, uint8_t *q, float *s)
{
    float a = 0.0f;
    for (int64_t c = 0; c < n; ++c) {
        float v = fabsf(oracle_bf16_to_f32(x[c]));
        if (v > a)                  /* false for NaN: NaN elements are skipped */
            a = v;
    }
    float sc = a / 448.0f;
    for (int64_t c = 0; c < n; ++c) {
        float v = oracle_bf16_to_f32(x[c]);
        if (a > 0.0f) {
            v = v / sc;
            if (v > 448.0f)
                v = 448.0f;
            if (v < -448.0f)
                v = -448.0f;
        }
        q[c] = isnan(v) ? nan_code_of(x[c]) : oracle_e4m3fn_rne(v);
    }
    *s = sc;
}

/* fp8 normal dispatch: each token row with at least one valid slot is
 * quantised once (H/group groups), and its (q, s) row is copied to every
 * destination row.  Q is [rows, H] bytes, S is [rows, H/group] fp32, row-major.
 * Returns -1 if group does not divide H. */
int32_t oracle_dispatch_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                            const int32_t *src2dst, int64_t group, uint8_t *Q,
                            float *S)
{
    if (group <= 0 || H % group != 0)
        return -1;
    int64_t G = H / group;
    uint8_t *qrow = (uint8_t *)malloc((size_t)(H > 0 ? H : 1));
    float *srow = (float *)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
    if (!qrow || !srow) {
        free(qrow);
        free(srow);
        return -2;
    }
    for (int64_t t = 0; t < T; ++t) {
        int any = 0;
        for (int32_t j = 0; j < k; ++j)
            any |= src2dst[t * k + j] >= 0;
        if (!any)
            continue;
        for (int64_t g = 0; g < G; ++g)
            oracle_quant_group_fp8(x + t * H + g * group, group, qrow + g * group,
                                   srow + g);
        for (int32_t j = 0; j < k; ++j) {
            int32_t d = src2dst[t * k + j];
            if (d < 0)
                continue;
            memcpy(Q + (int64_t)d * H, qrow, (size_t)H);
            memcpy(S + (int64_t)d * G, srow, sizeof(float) * (size_t)G);
        }
    }
    free(qrow);
    free(srow);
    return 0;
}

/* fp8 scale variants ([deepep.py], _DeepEPDispatcherImplNormal.dispatch_a:
 * the group quant takes column_major_scales, scale_tma_aligned and
 * scale_ue8m0 switches for DeepGEMM; _DeepEPDispatcherImplLowLatency.
 * _dispatch_core: round_scale / use_ue8m0 make DeepEP return int32-packed
 * UE8M0 scales).  Readings, as flags:
 *   UE8M0 (1):    the scale is the smallest power of two p >= 2^-127 with
 *                 448 * p >= amax, so x / p is exact and needs no clamp;
 *                 an all-zero group gets p = 2^-127
 *   COLMAJOR (2): the scales of each matrix of rows_per_mat rows are stored
 *                 group-major, [G][ld] with ld = rows_per_mat rounded up to
 *                 a multiple of 4 (16-byte aligned columns, as a TMA load
 *                 wants)
 *   PACKED (4):   (with UE8M0) the scale is stored as its exponent byte
 *                 log2(p) + 127, four consecutive groups per 32-bit word,
 *                 group g in byte g % 4 (little endian)
 * Without COLMAJOR the scales are row-major per destination row. */
enum { ORACLE_SCALE_UE8M0 = 1, ORACLE_SCALE_COLMAJOR = 2, ORACLE_SCALE_PACKED = 4 };

/* UE8M0 quantisation of one group: *p receives the power-of-two scale and
 * *p_exp its exponent. */
void oracle_quant_group_fp8_ue8m0(const uint16_t *x, int64_t n, uint8_t *q, float *p,
                                  int32_t *p_exp)
{
    double a = 0.0;
    for (int64_t c = 0; c < n; ++c) {
        double v = fabs((double)oracle_bf16_to_f32(x[c]));
        if (v > a)
            a = v;
    }
    /* the exponent stops at 127, the largest below the E8M0 NaN code: only
       an infinite amax (no finite bf16 needs more than 2^120) reaches it */
    int e = -127;
    while (e < 127 && ldexp(448.0, e) < a)
        ++e;
    float pf = (float)ldexp(1.0, e);
    for (int64_t c = 0; c < n; ++c) {
        float v = oracle_bf16_to_f32(x[c]) / pf;
        /* no clamp (exact scaling): +-inf x gives the NaN code with its sign */
        q[c] = isnan(v) ? nan_code_of(x[c]) : oracle_e4m3fn_rne(v);
    }
    *p = pf;
    *p_exp = e;
}

/* Byte offset of the scale of (destination row, group g) in a scale buffer
 * of the given flags; G groups per row. */
static int64_t scale_offset(int32_t flags, int64_t row, int64_t g, int64_t G,
                            int64_t rows_per_mat)
{
    int packed = (flags & ORACLE_SCALE_PACKED) != 0;
    int64_t words = packed ? (G + 3) / 4 : G;          /* 32-bit words per row */
    if (flags & ORACLE_SCALE_COLMAJOR) {
        int64_t ld = (rows_per_mat + 3) / 4 * 4;
        int64_t mat = row / rows_per_mat, r = row % rows_per_mat;
        int64_t word = mat * words * ld + (packed ? g / 4 : g) * ld + r;
        return word * 4 + (packed ? g % 4 : 0);
    }
    return (row * words + (packed ? g / 4 : g)) * 4 + (packed ? g % 4 : 0);
}

/* Writes the scale of one group in the requested format. */
static void put_scale(uint8_t *S, int32_t flags, int64_t row, int64_t g, int64_t G,
                      int64_t rows_per_mat, float p, int32_t p_exp)
{
    int64_t off = scale_offset(flags, row, g, G, rows_per_mat);
    if (flags & ORACLE_SCALE_PACKED)
        S[off] = (uint8_t)(p_exp + 127);
    else
        memcpy(S + off, &p, sizeof p);
}

/* fp8 normal dispatch with a scale format: as oracle_dispatch_fp8 (group =
 * 128 for the kernels), scales written at scale_offset() of S (bytes).
 * rows_per_mat only matters for COLMAJOR.  Returns -1 for bad arguments. */
int32_t oracle_dispatch_fp8_fmt(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                                const int32_t *src2dst, int64_t group, int32_t flags,
                                int64_t rows_per_mat, uint8_t *Q, uint8_t *S)
{
    if (group <= 0 || H % group != 0 || rows_per_mat <= 0)
        return -1;
    if ((flags & ORACLE_SCALE_PACKED) && !(flags & ORACLE_SCALE_UE8M0))
        return -1;
    int64_t G = H / group;
    uint8_t *qrow = (uint8_t *)malloc((size_t)(H > 0 ? H : 1));
    float *prow = (float *)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
    int32_t *erow = (int32_t *)malloc(sizeof(int32_t) * (size_t)(G > 0 ? G : 1));
    if (!qrow || !prow || !erow) {
        free(qrow);
        free(prow);
        free(erow);
        return -2;
    }
    for (int64_t t = 0; t < T; ++t) {
        int any = 0;
        for (int32_t j = 0; j < k; ++j)
            any |= src2dst[t * k + j] >= 0;
        if (!any)
            continue;
        for (int64_t g = 0; g < G; ++g) {
            if (flags & ORACLE_SCALE_UE8M0) {
                oracle_quant_group_fp8_ue8m0(x + t * H + g * group, group, qrow + g * group,
                                             prow + g, erow + g);
            } else {
                oracle_quant_group_fp8(x + t * H + g * group, group, qrow + g * group, prow + g);
                erow[g] = 0;
            }
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t d = src2dst[t * k + j];
            if (d < 0)
                continue;
            memcpy(Q + (int64_t)d * H, qrow, (size_t)H);
            for (int64_t g = 0; g < G; ++g)
                put_scale(S, flags, d, g, G, rows_per_mat, prow[g], erow[g]);
        }
    }
    free(qrow);
    free(prow);
    free(erow);
    return 0;
}

/* Low-latency dispatch with fp8 rows: oracle_dispatch_ll's slots with the
 * rows quantised as oracle_dispatch_fp8_fmt (each expert's cap rows form one
 * scale matrix for COLMAJOR).  Returns the overflow flag, or -1. */
int32_t oracle_dispatch_ll_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                               const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                               int64_t cap, int64_t group, int32_t flags, uint8_t *Q,
                               uint8_t *S, int32_t *masked_m, int32_t *ll_src2dst)
{
    if (group <= 0 || H % group != 0 || cap <= 0)
        return -1;
    int32_t overflow = 0;
    int64_t *seen = (int64_t *)calloc((size_t)(L > 0 ? L : 1), sizeof(int64_t));
    if (!seen)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t i = t * k + j;
            int32_t e = local_expert(topk_ids[i], expert_begin, L);
            if (e < 0) {
                ll_src2dst[i] = -1;
                continue;
            }
            int64_t slot = seen[e]++;
            if (slot >= cap) {
                ll_src2dst[i] = -1;
                overflow = 1;
                continue;
            }
            ll_src2dst[i] = (int32_t)((int64_t)e * cap + slot);
        }
    for (int32_t e = 0; e < L; ++e)
        masked_m[e] = (int32_t)(seen[e] < cap ? seen[e] : cap);
    free(seen);
    int32_t rc = oracle_dispatch_fp8_fmt(x, T, H, k, ll_src2dst, group, flags, cap, Q, S);
    return rc < 0 ? rc : overflow;
}

/* ------------------------------------------------------------------------ */
/* Combine.                                                                  */
/* ------------------------------------------------------------------------ */

/* Weighted gather-combine ([0.4.4 diff], _DeepEPDispatcherImplNormal.combine_a:
 * the post-reorder takes the expert outputs, src2dst, topk_ids, topk_weights
 * and writes one row per token in the input dtype; [deepep.py],
 * _DeepEPDispatcherImplLowLatency._combine_core: low_latency_combine is given
 * topk_ids and topk_weights as well).
 *   out[t, h] = bf16_rne( fma chain over j ascending with map[t*k+j] >= 0 of
 *                         w[t, j] * Y[map[t*k+j], h], starting from +0 )
 * map is src2dst (normal) or ll_src2dst (low latency).  A map entry at or
 * beyond y_rows is treated as invalid; the count of such entries is
 * returned. */
int64_t oracle_combine(const uint16_t *Y, int64_t y_rows, int64_t H,
                       const int32_t *map, const float *w, int64_t T,
                       int32_t k, uint16_t *out)
{
    int64_t bad = 0;
    float *acc = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    if (!acc)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int32_t r = map[t * k + j];
            if (r < 0)
                continue;
            if ((int64_t)r >= y_rows) {
                ++bad;
                continue;
            }
            float wj = w[t * k + j];
            const uint16_t *yr = Y + (int64_t)r * H;
            for (int64_t h = 0; h < H; ++h)
                acc[h] = fmaf(wj, oracle_bf16_to_f32(yr[h]), acc[h]);
        }
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = oracle_bf16_rne(acc[h]);
    }
    free(acc);
    return bad;
}

/* The same weighted sum in fp64 without the final bf16 rounding; used only
 * to pin oracle_combine's fp32 result within one bf16 ulp. */
void oracle_combine_f64(const uint16_t *Y, int64_t y_rows, int64_t H,
                        const int32_t *map, const float *w, int64_t T,
                        int32_t k, double *out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t r = map[t * k + j];
            if (r < 0 || (int64_t)r >= y_rows)
                continue;
            double wj = (double)w[t * k + j];
            for (int64_t h = 0; h < H; ++h)
                out[t * H + h] += wj * (double)oracle_bf16_to_f32(Y[(int64_t)r * H + h]);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Host scalar.                                                              */
/* ------------------------------------------------------------------------ */

/* Low-latency grouped-GEMM hint ([deepep.py],
 * _DeepEPDispatcherImplLowLatency.dispatch_a; same formula in the
 * [0.4.4 diff]): expected_m = (T * group_size * k + num_experts) //
 * num_experts, with group_size the number of EP ranks. */
int64_t oracle_expected_m(int64_t T, int32_t num_ranks, int32_t k, int32_t E)
{
    if (E <= 0)
        return -1;
    return (T * (int64_t)num_ranks * (int64_t)k + (int64_t)E) / (int64_t)E;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the codecs (loops over the scalar definitions above, so   */
/* that the tests can sweep large value sets quickly).                       */
/* ------------------------------------------------------------------------ */

void oracle_bf16_rne_n(const float *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(v[i]);
}

void oracle_bf16_to_f32_n(const uint16_t *b, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f32(b[i]);
}

void oracle_e4m3fn_rne_n(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3fn_rne(v[i]);
}

void oracle_e4m3fn_to_f32_n(const uint8_t *b, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3fn_to_f32(b[i]);
}
