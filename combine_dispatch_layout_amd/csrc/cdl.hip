// cdl.hip -- HIP kernels and C ABI for the MI355X (gfx950) hot path of MoE
// token dispatch and combine on one expert-parallel rank.
//
// Pages cited (titles as in include/cdl.h):
//   [deepep.py]     SGLang token_dispatcher/deepep.py (main branch)
//   [0.4.4 diff]    sglang 0.4.4.post2 -> 0.4.4.post4, ep_moe/token_dispatcher.py
//   [flashinfer.py] SGLang token_dispatcher/flashinfer.py (main branch)
//
// The work is data movement plus a few ALU operations per element, so every
// kernel is bound by HBM bandwidth or by latency; there is no dense
// contraction and no MFMA.  Design points for CDNA4:
//   * Layout in two launches with no atomics across workgroups and no state
//     kept between calls: (A) per-superblock expert histograms; (B) every
//     workgroup (one wave per token) derives its own expert offsets from the
//     superblock counts plus a recount of the slots of its superblock that
//     precede it, then ranks its slots with wave ballots (__ballot /
//     popcount / readlane), so src2dst is deterministic and stable by flat
//     slot index.  Small batches (T*k <= 4096) skip (A): every workgroup
//     counts all slots itself.
//   * The permute fuses (B) with the row scatter (bf16, fp8, or into the
//     low-latency padded buffer): the layout's small loads are issued first,
//     then the token's row, so HBM reads are in flight while the offsets are
//     computed.
//   * Rows move as 16-byte lane accesses (buffer_load/store_dwordx4 through a
//     per-row buffer resource); a wave holds 14 chunks (224 bytes) of a row
//     per lane, one 7168-wide row, so a source row is read once whatever its
//     fan-out.  Each wave holds its token's k destinations in lanes and takes
//     them with readlane.
//   * Cache policies, measured: source rows are streamed in; dispatched bf16
//     rows are stored with the temporal policy so the combine finds them in
//     the Infinity Cache; the combine loads and stores non-temporally; fp8
//     rows and scales (read by no kernel here) are stored non-temporally.
//   * fp8 groups are quantised without a division (correctly rounded scale
//     and reciprocal from one correction step each, Markstein's correction
//     per element; checked exhaustively over bf16 inputs on the CPU).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "cdl.h"

// Scratch of cdl_permute_noalloc: the layout's superblock counts.  Each GPU
// holds its own copy of the array at its own address; host code uses that
// address (looked up with hipGetSymbolAddress), never the array's name.
static __device__ __align__(256) unsigned char scratch[CDL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kWave = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Rows are addressed through buffer resources: the row base and its length
// live in scalar registers, each lane adds a 32-bit offset, and the hardware
// range check returns zeros for loads past the row end and drops stores
// there, so no per-chunk bounds test or 64-bit lane address is needed.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kPolicyNT = 2;             // cache policy: non-temporal (streaming)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}
// Cache policy per access.  Measured on MI355X in the dispatch -> combine
// step: the dispatched rows are stored with the default (temporal) policy so
// that the next kernel finds them in the caches (the 256 MB Infinity Cache
// holds a 60 MB permuted buffer), while the combine, the last reader of those
// rows and the writer of rows nobody reads back soon, loads and stores
// non-temporally.
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ u32x4 buf_ld16_stream(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPolicyNT);
}
__device__ __forceinline__ void buf_st16(rsrc_t r, u32x4 v, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st16_stream(rsrc_t r, u32x4 v, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kPolicyNT);
}
__device__ __forceinline__ void buf_st8_stream(rsrc_t r, u32x2 v, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, kPolicyNT);
}
__device__ __forceinline__ int32_t buf_ld4(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: the compiler does not infer that threadIdx.x / 64 is uniform, and a
// buffer resource derived from a non-uniform value costs a readfirstlane
// loop around every access.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / 64); }

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values to a packed pair of bf16 patterns, round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).  NaN becomes the sign-kept quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b)
{
    uint16_t ha = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
    uint16_t hb = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
    if (a != a) ha = (ha & 0x8000u) | 0x7FC0u;
    if (b != b) hb = (hb & 0x8000u) | 0x7FC0u;
    return (uint32_t)ha | ((uint32_t)hb << 16);
}

// Two fp32 values (already clamped to [-448, 448]) to OCP E4M3FN bytes, round
// to nearest even: v_cvt_pk_fp8_f32, which on gfx950 produces the OCP format.
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four such values to one 32-bit word (bytes a, b, c, d from low to high):
// each v_cvt_pk_fp8_f32 writes one 16-bit half of its destination and keeps
// the other, so no masking or shifting is needed.  The first conversion's
// "kept" half is a don't-care (it is overwritten by the second).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d)
{
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Non-finite bf16 patterns: exponent field all ones (Inf: mantissa 0, NaN:
// mantissa != 0), as the magnitude bits of a 16-bit half.
constexpr uint32_t kBf16ExpMask = 0x7F80u;

// The e4m3fn NaN code (S.1111.111) with the sign of the bf16 element x.
__device__ __forceinline__ uint32_t e4m3_nan_of(uint32_t x_bf16) { return ((x_bf16 >> 8) & 0x80u) | 0x7Fu; }

// Non-finite values among the 8 bf16 of a chunk: the exponent bits of every
// half masked and maximised as integers reach kBf16ExpMask iff one is Inf or
// NaN.
__device__ __forceinline__ bool chunk_has_nonfinite(u32x4 v)
{
    using u16x2 = unsigned short __attribute__((ext_vector_type(2)));
    const uint32_t m = 0x7F807F80u;
    const u16x2 e = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.x & m), __builtin_bit_cast(u16x2, v.y & m)),
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.z & m), __builtin_bit_cast(u16x2, v.w & m)));
    return (e.x > e.y ? e.x : e.y) == kBf16ExpMask;
}

__device__ __forceinline__ int32_t local_expert(int32_t id, int32_t expert_begin, int32_t L)
{
    // id - expert_begin in 64 bits: no overflow for any int32 pair
    int64_t e = (int64_t)id - (int64_t)expert_begin;
    return (e >= 0 && e < (int64_t)L) ? (int32_t)e : -1;
}

__device__ __forceinline__ void set_status(int32_t *status, int32_t bit)
{
    if (status) atomicOr(status, bit);
}

// ---------------------------------------------------------------------------
// fp8 group quantisation in the pair layout: a lane holds 32 contiguous bytes
// of a row (16 bf16, two 16-byte chunks: chunks 2l and 2l + 1 of a block of
// 128), so the 8 lanes of a DPP half row hold one group of 128 elements.  A
// lane computes its group's scale and reciprocal once per 16 elements, the
// group amax takes three DPP steps, and the 16 e4m3fn bytes leave in one
// 16-byte store.  Measured against one chunk per lane (16 lanes a group) at
// T = 4096, H = 7168, top-8 over 32 of 256 experts: fp8 permute 19.4 ->
// 18.0 us.
// ---------------------------------------------------------------------------

// Group amax.  Magnitudes of floats order like their bit patterns, so the
// maximum is taken on integers (no NaN canonicalisation, and the DPP moves
// fuse into the max): per lane over its 16 bf16 magnitudes in 16-bit halves,
// then over the 8 lanes of a half row (lanes 8j .. 8j+7): quad_perm swaps at
// distance 1 and 2 give each quad its maximum, row_half_mirror pairs the two
// quads.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax_step(uint32_t a)
{
    const uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, CTRL, 0xF, 0xF, false);
    return a > b ? a : b;
}
__device__ __forceinline__ uint32_t half_row_umax(uint32_t a)
{
    a = dpp_umax_step<0xB1>(a);    // quad_perm [1,0,3,2]
    a = dpp_umax_step<0x4E>(a);    // quad_perm [2,3,0,1]
    a = dpp_umax_step<0x141>(a);   // row_half_mirror: the other quad of the 8 lanes
    return a;
}

// Groups with amax >= 2^-96 (kFastQuotientMinBits) divide by the scale with one
// correctly rounded reciprocal y = 1/s per group and Markstein's correction
// step per element: q0 = x*y, the exact residual r = q0*s - x, q = q0 - r*y
// (the negation is a source modifier of the second fma; for x = +-0 the
// residual is +0 and q keeps the sign of x).  No clamp to [-448, 448]
// follows: with |x| <= amax, |q| <= 448 + 2^-15 (the float above 448, when
// fl(amax / 448) rounded down), and v_cvt_pk_fp8_f32 rounds every magnitude
// up to 464 to 448 (measured on gfx950; NaN only above 464), so the bytes are
// those of the clamped quotient.  An exhaustive check over every bf16 amax
// and every bf16 x with |x| <= amax (about 1.06e9 pairs,
// tests/fast_quotient_check.c) finds the e4m3fn code of this quotient equal
// to that of the correctly rounded x / s whenever amax >= 3.3e-32, and |q|
// never above 448 + 2^-15; below 2^-96 the exact path divides.
constexpr uint32_t kFastQuotientMinBits = 0x0F800000u;   // bits of 2^-96
static_assert(__builtin_bit_cast(float, kFastQuotientMinBits) == 0x1p-96f, "fast-path threshold");

// Exact path of a pair, taken by the whole wave when any of its groups is
// tiny (amax < 2^-96) or holds a non-finite value; it gives the same bytes as
// the fast paths for every other group.  Non-finite values (the pages say
// nothing of them; the oracle states the same reading):
//   * amax is taken over the group's non-NaN elements (an infinity counts);
//   * fp32 scales: s = fl(amax / 448) (infinite for an infinite amax), the
//     quotient x / s of a correctly rounded division (x / inf = +-0), clamped
//     to [-448, 448] with NaN passing through;
//   * power-of-two scales: the exponent is capped at 127, the largest below
//     the E8M0 NaN code;
//   * an element whose quotient is NaN (or infinite, with unclamped
//     power-of-two scaling) becomes the e4m3fn NaN code with x's sign.
__device__ __forceinline__ u32x4 quant_pair_exact(u32x4 a, u32x4 b, bool ue8m0, float *scale)
{
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[2 * i] = w[i] & 0xFFFFu;
        h[2 * i + 1] = w[i] >> 16;
    }
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t mag = h[e] & 0x7FFFu;
        if (mag <= kBf16ExpMask && mag > m) m = mag;
    }
    const float am = __uint_as_float(half_row_umax(m << 16));
    float q[16];
    if (ue8m0) {
        int e = -127;
        if (am > 0.0f) {
            int ex = 0;
            const float mt = frexpf(am, &ex);
            e = am == __builtin_huge_valf() ? 127 : ex - 9 + (mt > 0.875f ? 1 : 0);
            e = e < -127 ? -127 : e;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = ldexpf(__uint_as_float(h[i] << 16), -e);
        *scale = ldexpf(1.0f, e);
    } else {
        const float sc = am / 448.0f;                    // correctly rounded
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float x = __uint_as_float(h[i] << 16);
            const float d = am > 0.0f ? x / sc : x;
            q[i] = d > 448.0f ? 448.0f : (d < -448.0f ? -448.0f : d);
        }
        *scale = sc;
    }
    uint32_t bt[16];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        const uint32_t pk = pack2_e4m3(__builtin_isfinite(q[i]) ? q[i] : 0.0f,
                                       __builtin_isfinite(q[i + 1]) ? q[i + 1] : 0.0f);
        bt[i] = __builtin_isfinite(q[i]) ? (pk & 0xFFu) : e4m3_nan_of(h[i]);
        bt[i + 1] = __builtin_isfinite(q[i + 1]) ? (pk >> 8) : e4m3_nan_of(h[i + 1]);
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = bt[4 * i] | bt[4 * i + 1] << 8 | bt[4 * i + 2] << 16 | bt[4 * i + 3] << 24;
    return u32x4{o[0], o[1], o[2], o[3]};
}

// Returns the 16 e4m3fn bytes of the lane's pair; *scale receives the group
// scale (fp32, or the power of two of UE8M0 scales).  Lanes past the row
// (in_row false) never send the wave to the exact path; their bytes are not
// stored.
//
// Power-of-two (UE8M0) scales: p is the smallest power of two >= 2^-127 with
// 448 * p >= amax.  With amax = m * 2^ex, m in [0.5, 1) (frexp), that is
// 2^(ex - 9) when m <= 0.875 (448 = 0.875 * 2^9) and 2^(ex - 8) otherwise;
// x / p is then an exact power-of-two scaling and needs no clamp, and the
// scaled conversion takes the bf16 pairs as they are (8 instructions for 16
// elements, against 16 unpacks, 16 ldexp and 8 conversions).
__device__ __forceinline__ u32x4 quant_pair(u32x4 a, u32x4 b, bool ue8m0, bool in_row, float *scale)
{
    using u16x2 = unsigned short __attribute__((ext_vector_type(2)));
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    const uint32_t ab = half_row_umax((uint32_t)(m.x > m.y ? m.x : m.y) << 16);
    const uint32_t lo = ue8m0 ? 0u : kFastQuotientMinBits;
    // one exact path for the whole wave when any group needs it (a uniform
    // branch: the fast path below carries no exec-mask bookkeeping):
    // non-finite (ab >= the infinity pattern) or, for fp32 scales, tiny; one
    // unsigned range check
    const bool special = in_row && ab - lo >= (kBf16ExpMask << 16) - lo;
    if (__builtin_expect(__ballot(special) != 0, 0)) return quant_pair_exact(a, b, ue8m0, scale);
    const float am = __uint_as_float(ab);
    if (ue8m0) {
        int ex = 0;
        const float mt = frexpf(am, &ex);
        int e = am > 0.0f ? ex - 9 + (mt > 0.875f ? 1 : 0) : -127;
        e = e < -127 ? -127 : e;
        *scale = ldexpf(1.0f, e);
        // v_cvt_scalef32_pk_fp8_bf16 gives the e4m3fn codes, round to
        // nearest even, of two bf16 x / 2^E, E the scale's exponent field
        // read as an E8M0 code (field 0: 2^-127); here |x / 2^e| <= 448.
        // Checked on gfx950 against every bf16 x for E = -127, -126, -20,
        // -3, 0, 3, 20, 127: identical codes (the one other case, |x / 2^E|
        // = 464 exactly, gives 448's code and never occurs here).
        using v2i16 = short __attribute__((ext_vector_type(2)));
        using v2bf16 = __bf16 __attribute__((ext_vector_type(2)));
        const float p = __uint_as_float((uint32_t)(e + 127) << 23);
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v2i16 h = {0, 0};
            h = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h, __builtin_bit_cast(v2bf16, w[2 * i]), p, false);
            h = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h, __builtin_bit_cast(v2bf16, w[2 * i + 1]), p, true);
            o[i] = __builtin_bit_cast(uint32_t, h);
        }
        return u32x4{o[0], o[1], o[2], o[3]};
    }
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
    float q[16];
    // fp32 scales: sc = fl(amax / 448) = fl((amax * 2^-6) / 7) by one correction step
    // with fl(1/7); y = fl(1 / sc) by one correction step from v_rcp_f32
    // (within 1 ulp); both exact for every bf16 amax >= 2^-96 (exhaustive
    // CPU check)
    const float c7 = 1.0f / 7.0f;
    const float t = am * 0x1p-6f;
    const float s0 = t * c7;
    const float sc = fmaf(fmaf(-s0, 7.0f, t), c7, s0);
    const float r0 = __builtin_amdgcn_rcpf(sc);
    const float y = fmaf(fmaf(-sc, r0, 1.0f), r0, r0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float q0 = f[i] * y;
        q[i] = fmaf(-fmaf(q0, sc, -f[i]), y, q0);
    }
    *scale = sc;
    return u32x4{pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7]),
                 pack4_e4m3(q[8], q[9], q[10], q[11]), pack4_e4m3(q[12], q[13], q[14], q[15])};
}

// Per-tensor cast of one 16-byte chunk (8 bf16) to 8 e4m3fn bytes:
// e4m3_rne(clamp(fl(x / s), +-448)).  POW2: s is a power of two whose inverse
// inv is a normal float, so x * inv is the exact quotient; otherwise the
// quotient is a correctly rounded division.  A NaN quotient (x NaN) becomes
// the e4m3fn NaN code with x's sign, an infinite one saturates; POW2 leaves
// those to a wave-uniform branch taken only when the chunks of the wave hold
// a non-finite value.
template <bool POW2>
__device__ __forceinline__ u32x2 cast_chunk_fp8(u32x4 v, float s, float inv)
{
    const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                        bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float q[8];
    if (!POW2 || __builtin_expect(__ballot(chunk_has_nonfinite(v)) != 0, 0)) {
        const uint32_t h[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                               v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float d = POW2 ? f[e] * inv : f[e] / s;
            q[e] = d > 448.0f ? 448.0f : (d < -448.0f ? -448.0f : d);
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const uint32_t p = pack2_e4m3(q[e] == q[e] ? q[e] : 0.0f, q[e + 1] == q[e + 1] ? q[e + 1] : 0.0f);
            b[e] = q[e] == q[e] ? (p & 0xFFu) : e4m3_nan_of(h[e]);
            b[e + 1] = q[e + 1] == q[e + 1] ? (p >> 8) : e4m3_nan_of(h[e + 1]);
        }
        return u32x2{b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24, b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = __builtin_amdgcn_fmed3f(f[e] * inv, -448.0f, 448.0f);
    return u32x2{pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7])};
}

// Where fp8 rows and their scales go.  Scale layouts (CDL_FP8_SCALE_*):
// row-major fp32 [rows][groups]; column-major: every rows_per_mat rows form a
// matrix stored [groups][ld], ld = rows_per_mat rounded up to 4; packed: the
// exponent byte log2(p) + 127, four groups per 32-bit word (group g in byte
// g % 4), in either order.
struct Fp8Out {
    u32x2 *q;              // e4m3fn rows, 8 bytes per 16-byte input chunk
    uint8_t *s;            // scale buffer
    int32_t flags;
    int64_t groups;        // scales per row (H / 128)
    int64_t rows_per_mat;  // rows of one column-major matrix
    int64_t ld;            // column stride of a column-major matrix
};

// ---------------------------------------------------------------------------
// layout plan
// ---------------------------------------------------------------------------

constexpr int kMaxChunks = 14;          // 16-byte chunks a lane holds per pass (bf16 rows): 14 x 64 = 896, one row at H = 7168
constexpr int kMaxChunksFp8 = 14;       // the same for rows quantised on the way (one pass at
                                        // H = 7168, 7 pairs of chunks per lane)
constexpr int kCountThreads = 256;
constexpr int kSelfCountIds = 8;        // ids per thread when workgroups count every slot
constexpr int kFp8WavesSmall = 7;       // waves per token for fp8 rows of small self-counted
                                        // batches (2 chunks per lane each)

struct Plan {
    int64_t n;            // slots, T * k
    int tpb;              // tokens per permute workgroup (one wave each)
    int64_t nblocks;      // permute workgroups, ceil(T / tpb)
    int64_t sbb;          // permute workgroups per superblock
    int64_t S;            // superblocks
    int64_t sb_slots;     // slots per superblock
};

// Tokens per workgroup: enough workgroups to fill the chip (about 512) for
// small batches, max_tpb tokens for large ones (8, 512 threads, for bf16
// rows; 4 for fp8 rows, measured 23.1 -> 22.1 us at T = 4096, H = 7168,
// where 8 is best for bf16, 39.6 against 43.4 us per step).  Superblock
// size: the power of two that balances the superblock counts every workgroup
// reads (S * L) against the slots it may recount (sbb * tpb * k).
inline Plan make_plan(int64_t T, int32_t k, int32_t L, int max_tpb)
{
    Plan p;
    p.n = T * k;
    int tpb = 1;
    while (tpb < max_tpb && (T + tpb - 1) / tpb > 512) tpb *= 2;
    // a batch small enough for every workgroup to count all of its slots:
    // enough tokens per workgroup that the ids fit the one batch of loads
    // issued before the rows (kSelfCountIds per thread)
    if (p.n <= (int64_t)kSelfCountIds * kWave * 8)
        while (p.n > (int64_t)kSelfCountIds * kWave * tpb) tpb *= 2;
    p.tpb = tpb;
    p.nblocks = (T + tpb - 1) / tpb;
    const int64_t bs = (int64_t)tpb * k;
    int64_t best_sbb = 1, best_cost = INT64_MAX;
    for (int64_t sbb = 1; sbb <= (p.nblocks > 0 ? p.nblocks : 1); sbb *= 2) {
        const int64_t S = (p.nblocks + sbb - 1) / sbb;
        const int64_t cost = S * (int64_t)L + (sbb - 1) * bs;
        if (cost < best_cost) {
            best_cost = cost;
            best_sbb = sbb;
        }
    }
    p.sbb = best_sbb;
    p.S = (p.nblocks + best_sbb - 1) / best_sbb;
    p.sb_slots = best_sbb * bs;
    return p;
}

// ---------------------------------------------------------------------------
// layout kernel A: superblock histograms
// ---------------------------------------------------------------------------

// sb_counts[s][e] = number of valid slots of local expert e in superblock s
// (an LDS histogram; counts are order independent).  Each thread loads a batch
// of kCountBatch ids before touching the histogram, so one superblock costs
// one memory latency per batch rather than one per id.
constexpr int kCountBatch = 8;

__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(
    const int32_t *__restrict__ ids, int64_t n, int64_t sb_slots, int32_t expert_begin, int32_t L,
    int32_t *__restrict__ sb_counts)
{
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < L; e += kCountThreads) hist[e] = 0;
    const int64_t begin = (int64_t)blockIdx.x * sb_slots;
    const int64_t end = begin + sb_slots < n ? begin + sb_slots : n;
    // ids of the superblock through a buffer resource: loads past its end
    // return 0 without a branch (their slots are masked below)
    const rsrc_t r = make_rsrc(ids + begin, (uint32_t)((end > begin ? end - begin : 0) * 4));
    for (int64_t b0 = begin; b0 < end; b0 += (int64_t)kCountThreads * kCountBatch) {
        int32_t raw[kCountBatch], le[kCountBatch];
#pragma unroll
        for (int q = 0; q < kCountBatch; ++q)
            raw[q] = buf_ld4(r, (uint32_t)(q * kCountThreads + threadIdx.x) * 4u, (uint32_t)((b0 - begin) * 4));
#pragma unroll
        for (int q = 0; q < kCountBatch; ++q) {
            const int64_t i = b0 + q * kCountThreads + threadIdx.x;
            le[q] = i < end ? local_expert(raw[q], expert_begin, L) : -1;
        }
        if (b0 == begin) __syncthreads();            // histogram zeroed
#pragma unroll
        for (int q = 0; q < kCountBatch; ++q)
            if (le[q] >= 0) atomicAdd(&hist[le[q]], 1);
    }
    if (end <= begin) __syncthreads();
    __syncthreads();
    int32_t *row = sb_counts + (int64_t)blockIdx.x * L;
    for (int e = threadIdx.x; e < L; e += kCountThreads) row[e] = hist[e];
}

// fp8 rows and scales are stored non-temporally: nothing in this library
// reads them back (unlike the bf16 permuted rows, which the combine re-reads
// from the Infinity Cache), and back-to-back fp8 dispatches measured faster
// without the dirty lines they would leave there (scatter 20.7 -> 18.9 us at
// T = 4096, H = 7168).  Column-major scales are the exception (see
// store_scales_pairs).
//
// fp8 row passes hold the row in the pair layout (quant_pair): a pass of a
// wave starting at chunk c0 spans NCH * 64 chunks, and lane l keeps chunks
// c0 + 128p + 2l and c0 + 128p + 2l + 1 in v[2p] and v[2p + 1].  The first
// kFp8AheadPairs pairs are loaded before the layout or the wait for it; the
// rest follow as pairs are quantised.  Row offsets sit in the VGPR operand,
// which the range check covers.
constexpr int kFp8AheadPairs = 4;
template <int NCH>
__device__ __forceinline__ void load_fp8_first_parts(u32x4 (&v)[NCH], rsrc_t xr, int lane, int64_t c0)
{
    static_assert(NCH % 2 == 0, "a pass holds whole pairs");
    const uint32_t voff = (uint32_t)lane * 32u + (uint32_t)(c0 * 16);
#pragma unroll
    for (int p = 0; p < NCH / 2; ++p) {
        if (p < kFp8AheadPairs) {
            v[2 * p] = buf_ld16(xr, voff + p * 2048, 0);
            v[2 * p + 1] = buf_ld16(xr, voff + p * 2048 + 16u, 0);
        }
    }
}

// The scales of a pass in the pair layout starting at chunk c0: lane 8j + p
// (p < NP) holds the fp32 bits of the scale of group c0 / 16 + 8p + j, so a
// destination row's scales of the pass leave in one store of up to 56 lanes
// (dword stores; byte stores of the exponent e + 127 of the power of two
// 2^e >= 2^-127, its bits >> 23, when packed).  Column-major scales are
// stored with the temporal policy: each lane writes one word of a line that
// 32 rows share, and the L2 merges those pieces before they reach memory;
// streamed, every piece went out by itself (T = 4096, H = 7168, top-8 over
// 32 of 256 experts, padded to 128: packed UE8M0 22.6 -> 20.2 us, fp32
// 29.9 -> 21.5 us; row-major 19.2 us).
template <int NP>
__device__ __forceinline__ void store_scales_pairs(uint32_t sw, int lane, int64_t c0, int64_t chunks,
                                                   const Fp8Out &o, int32_t dlane, uint64_t dmask)
{
    const int pp = lane & 7;
    const int64_t g = c0 / 16 + (int64_t)pp * 8 + (lane >> 3);
    const bool active = pp < NP && g < chunks / 16;
    const bool packed = (o.flags & CDL_FP8_SCALE_PACKED) != 0;
    const bool colmajor = (o.flags & CDL_FP8_SCALE_COLMAJOR) != 0;
    const uint32_t word = packed ? sw >> 23 : sw;
    const int64_t words = packed ? (o.groups + 3) / 4 : o.groups;
    const int64_t col = packed ? g / 4 : g;
    const int64_t lane_off = colmajor ? col * o.ld * 4 + (packed ? (g & 3) : 0) : (packed ? g : g * 4);
    for (uint64_t m = dmask; m; m &= m - 1) {
        const int32_t dst = __builtin_amdgcn_readlane(dlane, (int)__builtin_ctzll(m));
        int64_t base;
        if (colmajor) {
            const int32_t rpm = (int32_t)o.rows_per_mat;
            const int32_t mat = dst / rpm;
            base = ((int64_t)mat * words * o.ld + (dst - mat * rpm)) * 4;
        } else {
            base = (int64_t)dst * words * 4;
        }
        if (!active) continue;
        uint8_t *q = o.s + base + lane_off;
        if (colmajor) {
            if (packed)
                *q = (uint8_t)word;
            else
                *reinterpret_cast<uint32_t *>(q) = word;
        } else if (packed) {
            __builtin_nontemporal_store((uint8_t)word, q);
        } else {
            __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(q));
        }
    }
}

// A row pass of fp8 rows, pair by pair: pair p is quantised and stored to
// every destination before pair p + 1, and the load of pair
// p + kFp8AheadPairs is issued as soon as pair p is quantised (its registers
// are free then).  The caller loads the first pairs (load_fp8_first_parts).
// The wave thus keeps kFp8AheadPairs pairs of loads in flight, and its
// stores drain while it quantises the next pairs.  Destinations: bit j of
// dmask is set when slot j's row (lane j of dlane) is stored; only those are
// visited.  Pairs past the row end are quantised all the same (their loads
// return zeros) and their stores fall outside the range: a branch around
// them would leave the compiler's wait counts for the loads in flight
// inexact (see below).
template <int NCH>
__device__ __forceinline__ void quant_store_pass(u32x4 (&v)[NCH], int lane, int64_t c0, int64_t chunks,
                                                 const Fp8Out &o, bool ue8m0, int32_t dlane,
                                                 uint64_t dmask, rsrc_t xr)
{
    constexpr int NP = NCH / 2;
    uint32_t sw = 0;
    const uint32_t q_bytes = (uint32_t)(chunks * 8);
    // The first two destinations get a fixed number of store instructions
    // per pair (a missing one stores through an empty range: no memory
    // access), so the compiler's wait counts for the pair loads still in
    // flight stay exact; with a loop of unknown length before them it must
    // assume the loop stored nothing, and each wait for a load would also
    // wait for the stores issued since.  More destinations (a tenth of the
    // tokens of top-8 over 32 of 256 experts) take a loop after the two.
    const uint64_t m1 = dmask & (dmask - 1);
    const int32_t d0 = dmask ? __builtin_amdgcn_readlane(dlane, (int)__builtin_ctzll(dmask)) : -1;
    const int32_t d1 = m1 ? __builtin_amdgcn_readlane(dlane, (int)__builtin_ctzll(m1)) : -1;
    const rsrc_t o0 = make_rsrc(o.q + (d0 >= 0 ? (int64_t)d0 * chunks : 0), d0 >= 0 ? q_bytes : 0u);
    const rsrc_t o1 = make_rsrc(o.q + (d1 >= 0 ? (int64_t)d1 * chunks : 0), d1 >= 0 ? q_bytes : 0u);
    const uint64_t rest = m1 & (m1 - 1);
    const uint32_t loff = (uint32_t)lane * 32u + (uint32_t)(c0 * 16);
    // 16-byte stores take their whole offset in the VGPR operand (see
    // combine_rows_pipe)
    const uint32_t soff = (uint32_t)lane * 16u + (uint32_t)(c0 * 8);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        float sc;
        const u32x4 q = quant_pair(v[2 * p], v[2 * p + 1], ue8m0, c0 + p * 128 + 2 * lane < chunks, &sc);
        // lane 8j + p keeps the scale of pair p (see store_scales_pairs)
        sw = (lane & 7) == p ? __float_as_uint(sc) : sw;
        if (p + kFp8AheadPairs < NP) {
            v[2 * (p + kFp8AheadPairs)] = buf_ld16(xr, loff + (p + kFp8AheadPairs) * 2048, 0);
            v[2 * (p + kFp8AheadPairs) + 1] = buf_ld16(xr, loff + (p + kFp8AheadPairs) * 2048 + 16u, 0);
        }
        buf_st16_stream(o0, q, soff + p * 1024, 0);
        buf_st16_stream(o1, q, soff + p * 1024, 0);
        for (uint64_t m = rest; m; m &= m - 1) {
            const int32_t dst = __builtin_amdgcn_readlane(dlane, (int)__builtin_ctzll(m));
            const rsrc_t oq = make_rsrc(o.q + (int64_t)dst * chunks, q_bytes);
            buf_st16_stream(oq, q, soff + p * 1024, 0);
        }
    }
    store_scales_pairs<NP>(sw, lane, c0, chunks, o, dlane, dmask);
}

// ---------------------------------------------------------------------------
// layout kernel B (+ fused row scatter): the permute
// ---------------------------------------------------------------------------

enum PermuteMode {
    kLayoutOnly = 0, kRowsBf16 = 1, kRowsFp8 = 2, kRowsLL = 3, kRowsLLFp8 = 4,
    kRowsFp8Tensor = 5,   // per-tensor fp8 cast (no per-row scales), scale from the device
    kRowsFp8Cast1 = 6     // the same with no scale given (s = 1): no division
};

// Block-wide exclusive scan of one int32 per thread (NW waves).
// Inclusive prefix sum over the 64 lanes of a wave with DPP moves only: shifts
// by 1, 2, 4 and 8 lanes inside each row of 16, then row 0's total added to
// row 1 and row 2's to row 3 (row_bcast:15), then rows 0-1's total to rows
// 2-3 (row_bcast:31).  Lanes whose source is outside the row or masked keep
// the 0 passed as the old value.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2, 3
    return v;
}

template <int NW>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t *lds_waves, int32_t *total)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = wave_id();
    int32_t incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) lds_waves[w] = incl;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int32_t s = lds_waves[i];
        if (i < w) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

struct PermuteArgs {
    const int32_t *ids;
    int64_t T;
    int32_t k;
    int32_t expert_begin;
    int32_t L;
    const int32_t *sb_counts;
    int64_t S;
    int32_t sbb_shift;    // log2 of the permute workgroups per superblock
    int64_t sb_slots;
    int32_t alignment;    // expert segments padded to multiples of this
    int32_t *counts;
    int64_t *seg_indptr;
    int32_t *src2dst;
    int32_t *reorder;
    int64_t reorder_cap;  // entries of reorder
    // rows
    const u32x4 *x;
    int64_t chunks;       // H / 8
    u32x4 *out;           // bf16 rows
    Fp8Out fp8;           // fp8 rows and scales
    const float *tensor_scale;   // per-tensor fp8 cast: device scalar, NULL = 1
    int64_t cap_rows;
    int32_t *status;
    // small batches: every workgroup counts all slots itself (no count kernel)
    int32_t self_count;
    // low-latency modes: rows go to [L, ll_cap, H]
    int64_t ll_cap;
    int32_t *masked_m;
    int32_t *ll_src2dst;
};

// fp8 rows of one pass held in registers (the split permute's row waves and
// the fp8 scatter from a given layout).
// The row arrives in the pair layout of load_fp8_first_parts (v[2p] and
// v[2p + 1] hold pair p), kFp8AheadPairs pairs ahead of the conversion, and
// the e4m3fn bytes of every pair (16 per lane) stay in q until the caller
// stores them with store_held_row.  Holding the row until its last pair is
// converted, instead of storing each pair as soon as it is ready
// (quant_store_pass), keeps the stores out of the waits for the later
// pairs' loads (fp8 scatter at T = 4096, H = 7168: 17.1 -> 15.8 us).
constexpr int kHeldPairs = kMaxChunksFp8 / 2;   // 128-chunk blocks of a row, one pair per lane each

// Converts the pairs as they arrive (groups of 128 with their scale in sw,
// lane 8j + p holding group 8p + j's, for kRowsFp8; the per-tensor cast
// otherwise) and issues the loads of the later pairs as registers free
// up.  Blocks past the row (H < 7168) are neither converted nor stored.
template <int MODE>
__device__ __forceinline__ void convert_held_row(u32x4 (&v)[2 * kHeldPairs], rsrc_t xr, int lane,
                                                 int64_t chunks, bool ue8m0, float cast_s,
                                                 float cast_inv, u32x4 (&q)[kHeldPairs], uint32_t &sw)
{
    constexpr bool kGroups = MODE == kRowsFp8;
    // the whole offset sits in the VGPR operand, which the range check covers
    const uint32_t voff = (uint32_t)lane * 32u;
#pragma unroll
    for (int p = 0; p < kHeldPairs; ++p) {
        if ((int64_t)p * 128 < chunks) {
            if constexpr (kGroups) {
                float sc;
                q[p] = quant_pair(v[2 * p], v[2 * p + 1], ue8m0, (int64_t)p * 128 + 2 * lane < chunks, &sc);
                sw = (lane & 7) == p ? __float_as_uint(sc) : sw;
            } else if (MODE == kRowsFp8Cast1 || cast_inv != 0.0f) {
                const u32x2 c0 = cast_chunk_fp8<true>(v[2 * p], cast_s, cast_inv);
                const u32x2 c1 = cast_chunk_fp8<true>(v[2 * p + 1], cast_s, cast_inv);
                q[p] = u32x4{c0.x, c0.y, c1.x, c1.y};
            } else {
                const u32x2 c0 = cast_chunk_fp8<false>(v[2 * p], cast_s, cast_inv);
                const u32x2 c1 = cast_chunk_fp8<false>(v[2 * p + 1], cast_s, cast_inv);
                q[p] = u32x4{c0.x, c0.y, c1.x, c1.y};
            }
        } else {
            q[p] = u32x4{0u, 0u, 0u, 0u};
        }
        if (p + kFp8AheadPairs < kHeldPairs) {
            v[2 * (p + kFp8AheadPairs)] = buf_ld16(xr, voff + (p + kFp8AheadPairs) * 2048, 0);
            v[2 * (p + kFp8AheadPairs) + 1] = buf_ld16(xr, voff + (p + kFp8AheadPairs) * 2048 + 16u, 0);
        }
    }
}

// The held row to every destination in dmask (lane j < k holds slot j's row
// in dlane), then its scales when GROUPS.
template <bool GROUPS>
__device__ __forceinline__ void store_held_row(const u32x4 (&q)[kHeldPairs], uint32_t sw, int lane,
                                               int64_t chunks, const Fp8Out &o, int32_t dlane,
                                               uint64_t dmask)
{
    const uint32_t q_bytes = (uint32_t)(chunks * 8);
    for (uint64_t m = dmask; m; m &= m - 1) {
        const int32_t dst = __builtin_amdgcn_readlane(dlane, (int)__builtin_ctzll(m));
        const rsrc_t oq = make_rsrc(o.q + (int64_t)dst * chunks, q_bytes);
        // the whole offset in the VGPR operand (see combine_rows_pipe)
#pragma unroll
        for (int p = 0; p < kHeldPairs; ++p)
            if ((int64_t)p * 128 < chunks) buf_st16_stream(oq, q[p], (uint32_t)lane * 16u + p * 1024, 0);
    }
    if constexpr (GROUPS) store_scales_pairs<kHeldPairs>(sw, lane, 0, chunks, o, dlane, dmask);
}

// The per-tensor scale s of the fp8 cast modes (the device scalar, 1 when
// none is given) and, for a power of two whose inverse is a normal float,
// that inverse (0 otherwise): such an s is applied by the exact product
// x * inv, any other by a correctly rounded division.
__device__ __forceinline__ void tensor_cast_scale(const PermuteArgs &a, float *s, float *inv)
{
    const float sv = a.tensor_scale ? *a.tensor_scale : 1.0f;
    const uint32_t sb = __float_as_uint(sv);
    const uint32_t ef = (sb >> 23) & 0xFFu;
    *s = sv;
    *inv = ((sb & 0x807FFFFFu) == 0 && ef >= 1 && ef <= 253) ? __uint_as_float((254u - ef) << 23) : 0.0f;
}

// Step 4 of the permutes: the wave's token row (its first pass already
// loaded into v; fp8 modes: its first pairs) goes to the destinations held
// in lanes (lane j < k: slot j's row, -1 for none), pass by pass; wave h of a
// token's WPT waves moves the chunks [h * NC * 64, (h + 1) * NC * 64) of
// each pass of WPT * NC * 64 chunks, starting at chunk c_first.
template <int MODE, int NC, int WPT>
__device__ __forceinline__ void store_token_rows(const PermuteArgs &a, u32x4 (&v)[NC], rsrc_t xr,
                                                 uint32_t voff, int64_t c_first, int32_t dlane,
                                                 int lane)
{
    constexpr bool kFp8Mode = MODE == kRowsFp8 || MODE == kRowsLLFp8;
    const int k = a.k;
    const uint32_t row_bytes = (uint32_t)(a.chunks * 16);
    float cast_s = 1.0f, cast_inv = 1.0f;      // kRowsFp8Cast1: s = 1
    if constexpr (MODE == kRowsFp8Tensor) tensor_cast_scale(a, &cast_s, &cast_inv);
    for (int64_t c0 = c_first; c0 < a.chunks; c0 += (int64_t)WPT * NC * kWave) {
        const uint32_t pass = (uint32_t)(c0 * 16);
        if (c0 > c_first && kFp8Mode) {
            load_fp8_first_parts(v, xr, lane, c0);
        } else if (c0 > c_first) {
#pragma unroll
            for (int u = 0; u < NC; ++u) v[u] = buf_ld16_stream(xr, voff, pass + u * kWave * 16);
        }
        if constexpr (MODE == kRowsFp8Tensor || MODE == kRowsFp8Cast1) {
            const uint32_t q_bytes = (uint32_t)(a.chunks * 8);
            auto row_dst = [&](int j, int u) -> int32_t {
                const int32_t dst = __builtin_amdgcn_readlane(dlane, j);
                if (dst >= 0 && (int64_t)dst >= a.cap_rows) {
                    if (u == 0 && c0 == 0 && lane == 0) set_status(a.status, CDL_STATUS_ROWS_OVERFLOW);
                    return -1;
                }
                return dst;
            };
            if (MODE == kRowsFp8Cast1 || cast_inv != 0.0f) {
                // exact scaling: the whole row is cast in place (the bytes
                // replace the first half of each chunk's registers), then
                // stored to every destination
#pragma unroll
                for (int u = 0; u < NC; ++u) {
                    const u32x2 c = cast_chunk_fp8<true>(v[u], cast_s, cast_inv);
                    v[u].x = c.x;
                    v[u].y = c.y;
                }
                for (int j = 0; j < k; ++j) {
                    const int32_t dst = row_dst(j, 0);
                    if (dst < 0) continue;
                    const rsrc_t o = make_rsrc(a.fp8.q + (int64_t)dst * a.chunks, q_bytes);
#pragma unroll
                    for (int u = 0; u < NC; ++u)
                        buf_st8_stream(o, u32x2{v[u].x, v[u].y}, (uint32_t)lane * 8u,
                                       (uint32_t)(c0 * 8) + u * kWave * 8);
                }
            } else {
                // a division per element: one chunk at a time, so that only
                // one chunk's division temporaries are live
#pragma unroll
                for (int u = 0; u < NC; ++u) {
                    const u32x2 c = cast_chunk_fp8<false>(v[u], cast_s, cast_inv);
                    for (int j = 0; j < k; ++j) {
                        const int32_t dst = row_dst(j, u);
                        if (dst < 0) continue;
                        const rsrc_t o = make_rsrc(a.fp8.q + (int64_t)dst * a.chunks, q_bytes);
                        buf_st8_stream(o, c, (uint32_t)lane * 8u, (uint32_t)(c0 * 8) + u * kWave * 8);
                    }
                }
            }
        } else if constexpr (!kFp8Mode) {
            for (int j = 0; j < k; ++j) {
                const int32_t dst = __builtin_amdgcn_readlane(dlane, j);
                if (dst < 0) continue;
                if ((int64_t)dst >= a.cap_rows) {
                    if (c0 == 0 && lane == 0) set_status(a.status, CDL_STATUS_ROWS_OVERFLOW);
                    continue;
                }
                const rsrc_t o = make_rsrc(a.out + (int64_t)dst * a.chunks, row_bytes);
#pragma unroll
                for (int u = 0; u < NC; ++u) buf_st16(o, v[u], voff, pass + u * kWave * 16);
            }
        } else {
            // rows at or beyond the capacity are dropped (reported once)
            const bool has = lane < k && dlane >= 0;
            const bool fits = has && (int64_t)dlane < a.cap_rows;
            if (c0 == 0 && __ballot(has && !fits) != 0 && lane == 0)
                set_status(a.status, CDL_STATUS_ROWS_OVERFLOW);
            const bool ue8m0 = (a.fp8.flags & CDL_FP8_SCALE_UE8M0) != 0;
            quant_store_pass(v, lane, c0, a.chunks, a.fp8, ue8m0, dlane, __ballot(fits), xr);
        }
    }
}

// One workgroup per TPB tokens, WPT waves per token (wave h of a token moves
// the chunks [h * NC * 64, (h + 1) * NC * 64) of each pass of its row).
//  0. every thread loads its first batch of layout operands, then the wave
//     of token t loads its row (all NC chunks per lane; the first pairs in
//     fp8 modes) if the token has a valid slot;
//  1. tot[e] = all valid slots of e; cur[e] = valid slots of e before this
//     workgroup's first slot (superblock counts of earlier superblocks plus a
//     recount of this superblock's earlier slots; with self_count, a count
//     of every slot);
//  2. exclusive scan over e of tot rounded up to the alignment gives
//     seg_indptr (workgroup 0 publishes counts and seg_indptr, and masked_m
//     in low-latency modes) and cur[e] += seg_indptr[e]; the padding rows of
//     expert e get reorder id -1 from workgroup e mod gridDim;
//  3. the workgroup's TPB*k slots are ranked 64 at a time, wave by wave in
//     slot order, with ballots; the leader of each expert match advances
//     cur[e]; dst = cur[e] + rank in the match;
//  4. each wave stores its row to its token's destinations (in low-latency
//     modes the padded-buffer rows e * cap + (dst - seg_indptr[e])).
// ALL_ROWS (small self-counted batches): every token's row is loaded at once,
// without first reading the token's ids to see whether it has a local slot,
// so the row and the ids arrive together instead of one after the other.
template <int TPB, int MODE, bool ALL_ROWS, int WPT>
__global__ __launch_bounds__(TPB *WPT *kWave) void permute_kernel(PermuteArgs a)
{
    constexpr int NW = TPB * WPT;         // waves
    constexpr int NT = NW * kWave;
    constexpr bool kFp8Mode = MODE == kRowsFp8 || MODE == kRowsLLFp8;
    constexpr bool kLLMode = MODE == kRowsLL || MODE == kRowsLLFp8;
    static_assert((kFp8Mode ? kMaxChunksFp8 : kMaxChunks) % WPT == 0, "chunks split over waves");
    constexpr int NC = (kFp8Mode ? kMaxChunksFp8 : kMaxChunks) / WPT;
    extern __shared__ int32_t lds[];
    const int L = a.L;
    int32_t *tot = lds;
    int32_t *cur = lds + L;
    int32_t *dsts = lds + 2 * L;          // [TPB * k]
    __shared__ int32_t scan_tmp[NW];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id();
    const int k = a.k;
    const int64_t blk = blockIdx.x;
    const int64_t t_begin = blk * TPB;
    const int64_t t_end = t_begin + TPB < a.T ? t_begin + TPB : a.T;
    const int64_t slot_begin = t_begin * k;
    const int nslots = (int)((t_end > t_begin ? t_end - t_begin : 0) * k);

    // 0. loads.  The layout's own operands go first (the first batch of
    //    superblock counts and of the recount, and the 64 slots this wave
    //    ranks), then the token's row.  A wave's loads complete in issue
    //    order, so the offsets below wait only for those small loads while
    //    the row is still in flight.
    constexpr int kBatch = 8;
    // self-counting: the first loop reads every id instead of superblock
    // counts, and nothing is recounted
    const bool self = a.self_count != 0;
    const int64_t n_all = a.T * k;
    const int64_t s_me = blk >> a.sbb_shift;
    const int64_t nsc = self ? n_all : a.S * L;
    const int64_t rc_begin = s_me * a.sb_slots;
    const int64_t nrc = self ? 0 : slot_begin - rc_begin;
    // WPT waves per token: wave h of token t moves the row chunks
    // [h * NC * 64, (h + 1) * NC * 64) of each pass of WPT * NC * 64 chunks
    const int64_t t = t_begin + wave / WPT;
    const int h = wave % WPT;
    const int64_t c_first = (int64_t)h * NC * kWave;
    const uint32_t hoff = (uint32_t)(c_first * 16);
    const bool real = t < a.T;
    // lane j < k holds the local expert of the wave's slot j: one vector load,
    // issued before the layout operands so that the wait for it (the row
    // loads below depend on it) waits for no other load.  It replaced k
    // dependent scalar loads, which took up to 5 us under the row traffic of
    // the other waves (T = 4096, H = 7168: 38.9 -> 38.2 us per step).  A wave
    // past the last token reads an empty range, whose zeros are not ids.
    int32_t e_lane = -1;
    if (MODE != kLayoutOnly && (kLLMode || !ALL_ROWS)) {
        const rsrc_t r_tok = make_rsrc(a.ids + (real ? t * k : 0), real ? (uint32_t)k * 4u : 0u);
        const int32_t id_lane = buf_ld4(r_tok, (uint32_t)lane * 4u, 0);
        // keep it first: scheduled after the layout loads, the wait for it
        // waited for them too (38.5 against 38.2 us per step)
        __builtin_amdgcn_sched_barrier(0);
        // a select, not a branch: the load must not sink into a branch
        const int32_t le = local_expert(id_lane, a.expert_begin, L);
        e_lane = ((lane < k) & real) ? le : -1;
    }
    const rsrc_t r_sc = self ? make_rsrc(a.ids, (uint32_t)(n_all * 4)) : make_rsrc(a.sb_counts, (uint32_t)(nsc * 4));
    const rsrc_t r_rc = make_rsrc(a.ids + rc_begin, (uint32_t)(nrc * 4));
    const rsrc_t r_my = make_rsrc(a.ids + slot_begin, (uint32_t)(nslots * 4));
    int32_t c[kBatch], id[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) c[q] = buf_ld4(r_sc, (uint32_t)(q * NT + tid) * 4u, 0);
#pragma unroll
    for (int q = 0; q < kBatch; ++q) id[q] = buf_ld4(r_rc, (uint32_t)(q * NT + tid) * 4u, 0);
    // nslots <= TPB * 64 (k <= 64), so wave w ranks exactly round w
    const int my_rel = wave * kWave + lane;
    const int32_t my_id = buf_ld4(r_my, (uint32_t)my_rel * 4u, 0);

    // low latency: the local experts of the slots, for the padded rows
    const int32_t ll_e = e_lane;
    // tok_valid: the token's row is loaded and stored to its destinations
    bool tok_valid = false;
    if (MODE != kLayoutOnly && real) tok_valid = ALL_ROWS ? true : __ballot(e_lane >= 0) != 0;
    u32x4 v[NC];
    const uint32_t row_bytes = (uint32_t)(a.chunks * 16);
    const uint32_t voff = (uint32_t)lane * 16u;
    // The row loads are issued on every path: a wave whose token has no
    // local slot (or lies past the last token) gets an empty range, whose
    // loads return 0 and touch no memory.  The compiler's wait counts for the
    // layout operands above are then exact; with the loads behind a branch it
    // had to assume the path without them, and the layout waited for part of
    // every row (measured at T = 4096, H = 7168: 39.1 -> 38.9 us per step).
    const rsrc_t xr = make_rsrc(a.x + (tok_valid ? t * a.chunks : 0), tok_valid ? row_bytes : 0u);
    if (MODE != kLayoutOnly) {
        if (kFp8Mode) {
            load_fp8_first_parts(v, xr, lane, c_first);
        } else {
            // source rows are read once: streaming loads leave the Infinity
            // Cache to the permuted rows, which the combine reads back
#pragma unroll
            for (int u = 0; u < NC; ++u) v[u] = buf_ld16_stream(xr, voff, hoff + u * kWave * 16);
        }
    }

    // 1. totals and offsets before this workgroup
    for (int e = tid; e < L; e += NT) {
        tot[e] = 0;
        cur[e] = 0;
    }
    __syncthreads();
    // superblock counts, kBatch per thread per round.  Entry idx = b0 +
    // q * NT + tid is superblock idx / L, expert idx % L: one 32-bit division
    // per thread, then advanced by NT entries at a time with adds (a 64-bit
    // division per entry cost about a hundred instructions on this path)
    uint32_t sb_s = 0, sb_e = 0;
    const uint32_t step_s = (uint32_t)NT / (uint32_t)L, step_e = (uint32_t)NT % (uint32_t)L;
    if (!self) {
        sb_s = (uint32_t)tid / (uint32_t)L;
        sb_e = (uint32_t)tid - sb_s * (uint32_t)L;
    }
    for (int64_t b0 = 0; b0 < nsc; b0 += (int64_t)NT * kBatch) {
        if (b0 > 0) {
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                c[q] = buf_ld4(r_sc, (uint32_t)(q * NT + tid) * 4u, (uint32_t)(b0 * 4));
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int64_t idx = b0 + q * NT + tid;
            if (self) {
                const int32_t e = idx < nsc ? local_expert(c[q], a.expert_begin, L) : -1;
                if (e >= 0) {
                    atomicAdd(&tot[e], 1);
                    if (idx < slot_begin) atomicAdd(&cur[e], 1);
                }
            } else {
                if (idx < nsc && c[q]) {
                    atomicAdd(&tot[sb_e], c[q]);
                    if ((int64_t)sb_s < s_me) atomicAdd(&cur[sb_e], c[q]);
                }
                sb_s += step_s;
                sb_e += step_e;
                if (sb_e >= (uint32_t)L) {
                    sb_e -= (uint32_t)L;
                    ++sb_s;
                }
            }
        }
    }
    // recount of this superblock's slots before the workgroup
    for (int64_t b0 = 0; b0 < nrc; b0 += (int64_t)NT * kBatch) {
        if (b0 > 0) {
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                id[q] = buf_ld4(r_rc, (uint32_t)(q * NT + tid) * 4u, (uint32_t)(b0 * 4));
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int32_t e = b0 + q * NT + tid < nrc ? local_expert(id[q], a.expert_begin, L) : -1;
            if (e >= 0) atomicAdd(&cur[e], 1);
        }
    }
    __syncthreads();

    // 2. scan over experts; each thread owns a run of consecutive experts
    {
        const int A = a.alignment;
        const int per = (L + NT - 1) / NT;
        const int e0 = tid * per;
        int32_t run = 0;
        for (int q = 0; q < per && e0 + q < L; ++q) run += (tot[e0 + q] + A - 1) / A * A;
        int32_t R = 0, excl = 0;
        if (ALL_ROWS && L <= kWave) {
            // thread e < L of wave 0 owns expert e: a DPP scan in that wave,
            // with no LDS round trips and no barriers.  Only small batches,
            // where the layout's latency is the step's: with the count
            // kernel's batches it measured 0.4 us slower per step (their row
            // stores then begin while other waves are still reading)
            if (wave == 0) {
                const int32_t incl = wave_inclusive_scan(run);
                excl = incl - run;
                R = __builtin_amdgcn_readlane(incl, kWave - 1);
            }
        } else {
            excl = block_exclusive_scan<NW>(run, scan_tmp, &R);
        }
        for (int q = 0; q < per && e0 + q < L; ++q) {
            const int e = e0 + q;
            const int32_t c = tot[e];
            const int32_t padded = (c + A - 1) / A * A;
            if (blk == 0) {
                a.counts[e] = c;
                a.seg_indptr[e] = excl;
                if (kLLMode) a.masked_m[e] = (int32_t)((int64_t)c < a.ll_cap ? c : a.ll_cap);
            }
            if (kLLMode) tot[e] = excl;          // segment start, for the padded rows
            cur[e] += excl;
            if (padded > c && (int64_t)(e % gridDim.x) == blk) {
                for (int64_t r = excl + c; r < excl + padded && r < a.reorder_cap; ++r) a.reorder[r] = -1;
            }
            excl += padded;
        }
        if (blk == 0 && tid == 0) {
            a.seg_indptr[L] = R;
            if ((int64_t)R > a.reorder_cap) set_status(a.status, CDL_STATUS_REORDER_OVERFLOW);
        }
    }
    __syncthreads();

    // 3. stable ranks, 64 slots per round in slot order
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int r0 = 0, rw = 0; r0 < nslots; r0 += kWave, ++rw) {
        if (wave == rw) {
            const int rel = r0 + lane;
            const int64_t i = slot_begin + rel;
            const int32_t e = rel < nslots ? local_expert(my_id, a.expert_begin, L) : -1;
            uint64_t pending = __ballot(e >= 0);
            int32_t dst = -1;
            while (pending) {
                const int leader = __builtin_ctzll(pending);
                const int32_t el = __builtin_amdgcn_readlane(e, leader);
                const uint64_t m = __ballot(e == el);
                const int32_t before = cur[el];
                if (e == el) dst = before + __popcll(m & lt_mask);
                if (lane == leader) cur[el] = before + __popcll(m);
                pending &= ~m;
            }
            if (rel < nslots) {
                a.src2dst[i] = dst;
                if (dst >= 0 && (int64_t)dst < a.reorder_cap) a.reorder[dst] = e;
                if (MODE != kLayoutOnly) dsts[rel] = dst;
            }
        }
        __syncthreads();
    }

    // 4. rows; lane j < k holds the destination of the token's slot j
    //    (readlane below: no memory access per destination)
    if (MODE == kLayoutOnly) return;
    int32_t dlane = -1;
    if (kLLMode) {
        // padded-buffer row e * ll_cap + (dst - seg_indptr[e]); rows past the
        // expert's capacity are dropped
        bool ovf = false;
        if (t < a.T && lane < k) {
            const int32_t d = dsts[(wave / WPT) * k + lane];
            if (d >= 0) {
                const int64_t slot = (int64_t)d - tot[ll_e];
                if (slot < a.ll_cap)
                    dlane = (int32_t)(ll_e * a.ll_cap + slot);
                else
                    ovf = true;
            }
            if (h == 0) a.ll_src2dst[t * k + lane] = dlane;
        }
        if (__ballot(ovf) != 0 && lane == 0) set_status(a.status, CDL_STATUS_LL_OVERFLOW);
    }
    if (!tok_valid) return;
    if (!kLLMode) dlane = lane < k ? dsts[(wave / WPT) * k + lane] : -1;
    store_token_rows<MODE, NC, WPT>(a, v, xr, voff, c_first, dlane, lane);
}

// The layout alone (cdl_dispatch_layout) for batches with superblock counts
// (the count kernel ran first): one wave per workgroup derives the
// destinations of its TPB tokens with wave-level operations only.  It loads
// the superblock counts, this superblock's slots before the workgroup
// (recount) and the workgroup's own slots in one batch, accumulates tot[e] /
// cur[e] with LDS atomics, scans the experts with DPP adds, and ranks the
// slots 64 at a time with ballots: no barrier, and every wait is for the
// layout's own operands.  (The all-waves kernel below spends its barriers
// waiting for its slowest wave; measured at T = 4096, top-8 over 32 of 256
// experts, the unfused layout + scatter + combine went 48.9 -> 48.5 us.
// Giving the row-moving permutes such a layout wave made them slower: their
// row stores then began while the other waves were still reading, 38.9 ->
// 40.7 us per prefill step, and the extra wave per workgroup of fp8 rows no
// longer fit the GPU at once.)
// The layout of workgroup blk (TPB tokens) by one wave: tot and cur are
// the wave's LDS arrays of L entries; with dsts != nullptr the destination
// of the workgroup's slot rel is also left in dsts[rel].
template <int TPB>
__device__ __forceinline__ void layout_one_wave(const PermuteArgs &a, int64_t blk, int32_t *tot,
                                                int32_t *cur, int32_t *dsts)
{
    constexpr int kLB = 16;              // layout operands per lane per batch
    const int L = a.L;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = a.k;
    const int64_t t_begin = blk * TPB;
    const int64_t t_end = t_begin + TPB < a.T ? t_begin + TPB : a.T;
    const int64_t slot_begin = t_begin * k;
    const int nslots = (int)((t_end > t_begin ? t_end - t_begin : 0) * k);
    const int64_t nblk = (a.T + TPB - 1) / TPB;

    {
        const int64_t s_me = blk >> a.sbb_shift;
        const int64_t nsc = a.S * L;
        const int64_t rc_begin = s_me * a.sb_slots;
        const int64_t nrc = slot_begin - rc_begin;
        const rsrc_t r_sc = make_rsrc(a.sb_counts, (uint32_t)(nsc * 4));
        const rsrc_t r_rc = make_rsrc(a.ids + rc_begin, (uint32_t)(nrc * 4));
        const rsrc_t r_my = make_rsrc(a.ids + slot_begin, (uint32_t)(nslots * 4));
        // every first batch is issued before any is used: one memory latency
        int32_t c[kLB], id[kLB], my[TPB];
#pragma unroll
        for (int q = 0; q < kLB; ++q) c[q] = buf_ld4(r_sc, (uint32_t)(q * kWave + lane) * 4u, 0);
#pragma unroll
        for (int q = 0; q < kLB; ++q) id[q] = buf_ld4(r_rc, (uint32_t)(q * kWave + lane) * 4u, 0);
        // nslots <= TPB * 64 (k <= 64): round r ranks slots [64 r, 64 r + 64)
#pragma unroll
        for (int r = 0; r < TPB; ++r) my[r] = buf_ld4(r_my, (uint32_t)(r * kWave + lane) * 4u, 0);
        for (int e = lane; e < L; e += kWave) {
            tot[e] = 0;
            cur[e] = 0;
        }
        // 1. totals and offsets before this workgroup.  Superblock-count entry
        //    idx = s * L + e is advanced 64 entries at a time with adds.
        uint32_t sb_s = (uint32_t)lane / (uint32_t)L, sb_e = (uint32_t)lane % (uint32_t)L;
        const uint32_t step_s = (uint32_t)kWave / (uint32_t)L, step_e = (uint32_t)kWave % (uint32_t)L;
        for (int64_t b0 = 0; b0 < nsc; b0 += (int64_t)kWave * kLB) {
            if (b0 > 0) {
#pragma unroll
                for (int q = 0; q < kLB; ++q)
                    c[q] = buf_ld4(r_sc, (uint32_t)(q * kWave + lane) * 4u, (uint32_t)(b0 * 4));
            }
#pragma unroll
            for (int q = 0; q < kLB; ++q) {
                if (b0 + q * kWave + lane < nsc && c[q]) {
                    atomicAdd(&tot[sb_e], c[q]);
                    if ((int64_t)sb_s < s_me) atomicAdd(&cur[sb_e], c[q]);
                }
                sb_s += step_s;
                sb_e += step_e;
                if (sb_e >= (uint32_t)L) {
                    sb_e -= (uint32_t)L;
                    ++sb_s;
                }
            }
        }
        for (int64_t b0 = 0; b0 < nrc; b0 += (int64_t)kWave * kLB) {
            if (b0 > 0) {
#pragma unroll
                for (int q = 0; q < kLB; ++q)
                    id[q] = buf_ld4(r_rc, (uint32_t)(q * kWave + lane) * 4u, (uint32_t)(b0 * 4));
            }
#pragma unroll
            for (int q = 0; q < kLB; ++q) {
                const int32_t e = b0 + q * kWave + lane < nrc ? local_expert(id[q], a.expert_begin, L) : -1;
                if (e >= 0) atomicAdd(&cur[e], 1);
            }
        }
        // 2. exclusive scan over the experts padded to the alignment, 64 at a
        //    time (DPP adds); workgroup 0 publishes counts and seg_indptr
        const int A = a.alignment;
        int32_t base = 0;
        for (int e0 = 0; e0 < L; e0 += kWave) {
            const int e = e0 + lane;
            const int32_t cnt = e < L ? tot[e] : 0;
            const int32_t padded = (cnt + A - 1) / A * A;
            const int32_t incl = wave_inclusive_scan(padded);
            const int32_t excl = base + incl - padded;
            if (e < L) {
                if (blk == 0) {
                    a.counts[e] = cnt;
                    a.seg_indptr[e] = excl;
                }
                cur[e] += excl;
                if (padded > cnt && (int64_t)(e % nblk) == blk) {
                    for (int64_t r = excl + cnt; r < excl + padded && r < a.reorder_cap; ++r) a.reorder[r] = -1;
                }
            }
            base += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        if (blk == 0 && lane == 0) {
            a.seg_indptr[L] = base;
            if ((int64_t)base > a.reorder_cap) set_status(a.status, CDL_STATUS_REORDER_OVERFLOW);
        }
        // 3. stable ranks, 64 slots per round in slot order; the leader of
        //    each expert match advances cur[e]
        const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
        for (int r = 0; r < TPB; ++r) {
            const int rel = r * kWave + lane;
            if (r * kWave >= nslots) break;
            const int32_t e = rel < nslots ? local_expert(my[r], a.expert_begin, L) : -1;
            uint64_t pending = __ballot(e >= 0);
            int32_t dst = -1;
            while (pending) {
                const int leader = __builtin_ctzll(pending);
                const int32_t el = __builtin_amdgcn_readlane(e, leader);
                const uint64_t m = __ballot(e == el);
                const int32_t before = cur[el];
                if (e == el) dst = before + __popcll(m & lt_mask);
                if (lane == leader) cur[el] = before + __popcll(m);
                pending &= ~m;
            }
            if (rel < nslots) {
                const int64_t i = slot_begin + rel;
                a.src2dst[i] = dst;
                if (dst >= 0 && (int64_t)dst < a.reorder_cap) a.reorder[dst] = e;
                if (dsts) dsts[rel] = dst;
            }
        }
    }
}

template <int TPB>
__global__ __launch_bounds__(kWave) void layout_wave_kernel(PermuteArgs a)
{
    extern __shared__ int32_t lds[];
    layout_one_wave<TPB>(a, blockIdx.x, lds, lds + a.L, nullptr);
}

// The fused fp8 permutes (groups of 128 with scales, or the per-tensor cast)
// for batches with superblock counts (the count kernel ran first) and rows
// of one pass (H <= 7168): TPB row waves and one layout wave per workgroup.
// A row wave loads its token's row as soon as it knows the token has a local
// slot, in the pair layout (quant_pair), and converts it pair by pair as the
// pairs arrive (the loads of the later pairs issued as the first pairs'
// registers free up), keeping the e4m3 bytes (16 per pair per lane) until the
// destinations are known.  The layout wave meanwhile derives the workgroup's
// destinations (layout_one_wave) into LDS.  After the workgroup's one
// barrier the row waves store their bytes and scales.  The quantisation,
// about a quarter of each SIMD's time, thus overlaps the layout's latency
// instead of following it.
template <int TPB, int MODE>
__global__ __launch_bounds__((TPB + 1) * kWave) void permute_fp8_split_kernel(PermuteArgs a)
{
    static_assert(MODE == kRowsFp8 || MODE == kRowsFp8Tensor || MODE == kRowsFp8Cast1, "fp8 row modes");
    constexpr bool kGroups = MODE == kRowsFp8;
    constexpr int NP = kHeldPairs;
    extern __shared__ int32_t lds[];
    const int L = a.L;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id();
    const int k = a.k;
    const int64_t blk = blockIdx.x;
    const int64_t t = blk * TPB + wave;
    const bool row_wave = wave < TPB;
    const bool real = row_wave && t < a.T;
    const Fp8Out &o = a.fp8;
    const bool ue8m0 = (o.flags & CDL_FP8_SCALE_UE8M0) != 0;
    bool tok_valid = false;
    u32x4 q[NP];
    uint32_t sw = 0;
    if (!row_wave) {
        layout_one_wave<TPB>(a, blk, lds, lds + L, lds + 2 * L);
    } else {
        // lane j < k holds the local expert of slot j; a wave past the last
        // token reads an empty range
        const rsrc_t r_tok = make_rsrc(a.ids + (real ? t * k : 0), real ? (uint32_t)k * 4u : 0u);
        const int32_t le = local_expert(buf_ld4(r_tok, (uint32_t)lane * 4u, 0), a.expert_begin, L);
        tok_valid = real && __ballot(lane < k && le >= 0) != 0;
        if (tok_valid) {
            const rsrc_t xr = make_rsrc(a.x + t * a.chunks, (uint32_t)(a.chunks * 16));
            u32x4 v[2 * NP];
            load_fp8_first_parts(v, xr, lane, 0);
            // per-tensor cast: the scale (kRowsFp8Tensor) read once per wave
            float cast_s = 1.0f, cast_inv = 1.0f;
            if constexpr (MODE == kRowsFp8Tensor) tensor_cast_scale(a, &cast_s, &cast_inv);
            convert_held_row<MODE>(v, xr, lane, a.chunks, ue8m0, cast_s, cast_inv, q, sw);
        }
    }
    __syncthreads();
    if (!tok_valid) return;
    const int32_t dlane = lane < k ? lds[2 * L + wave * k + lane] : -1;
    const bool has = lane < k && dlane >= 0;
    const bool fits = has && (int64_t)dlane < a.cap_rows;
    if (__ballot(has && !fits) != 0 && lane == 0) set_status(a.status, CDL_STATUS_ROWS_OVERFLOW);
    store_held_row<kGroups>(q, sw, lane, a.chunks, o, dlane, __ballot(fits));
}

// ---------------------------------------------------------------------------
// normal dispatch from a given layout: row scatter
// ---------------------------------------------------------------------------

constexpr int kRowTok = 4;                       // tokens (waves) per workgroup
constexpr int kRowThreads = kRowTok * kWave;

// One wave per token: the wave loads NC 16-byte chunks per
// lane of the row once, then stores them to every valid destination.
template <bool FP8>
__global__ __launch_bounds__(kRowThreads) void scatter_rows_kernel(
    const u32x4 *__restrict__ x, int64_t T, int64_t chunks, int32_t k,
    const int32_t *__restrict__ src2dst, u32x4 *__restrict__ out, Fp8Out fp8, int64_t cap_rows,
    int32_t *__restrict__ status)
{
    constexpr int NC = FP8 ? kMaxChunksFp8 : kMaxChunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowTok + wave_id();
    if (t >= T) return;
    // lane j < k holds the destination of slot j: one load for all slots,
    // then readlane per destination
    const int32_t dlane = lane < k ? src2dst[t * k + lane] : -1;
    if (__ballot(dlane >= 0) == 0) return;
    const uint32_t row_bytes = (uint32_t)(chunks * 16);
    const uint32_t voff = (uint32_t)lane * 16u;
    const rsrc_t xr = make_rsrc(x + t * chunks, row_bytes);
    for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)NC * kWave) {
        const uint32_t pass = (uint32_t)(c0 * 16);
        u32x4 v[NC];
        if (FP8) {
            load_fp8_first_parts(v, xr, lane, c0);
        } else {
#pragma unroll
            for (int u = 0; u < NC; ++u) v[u] = buf_ld16(xr, voff, pass + u * kWave * 16);
        }
        if (FP8) {
            const bool has = lane < k && dlane >= 0;
            const bool fits = has && (int64_t)dlane < cap_rows;
            if (c0 == 0 && __ballot(has && !fits) != 0 && lane == 0)
                set_status(status, CDL_STATUS_ROWS_OVERFLOW);
            const bool ue8m0 = (fp8.flags & CDL_FP8_SCALE_UE8M0) != 0;
            quant_store_pass(v, lane, c0, chunks, fp8, ue8m0, dlane, __ballot(fits), xr);
            continue;
        }
        for (int j = 0; j < k; ++j) {
            const int32_t dst = __builtin_amdgcn_readlane(dlane, j);
            if (dst < 0) continue;
            if (dst >= cap_rows) {
                if (c0 == 0 && lane == 0) set_status(status, CDL_STATUS_ROWS_OVERFLOW);
                continue;
            }
            const rsrc_t o = make_rsrc(out + (int64_t)dst * chunks, row_bytes);
#pragma unroll
            for (int u = 0; u < NC; ++u) buf_st16(o, v[u], voff, pass + u * kWave * 16);
        }
    }
}

// fp8 rows of one pass (H <= 7168) from a given layout: one wave per token
// holds its row (convert_held_row), then stores it to every destination.
// Without the occupancy bound the compiler kept every pair's temporaries
// live at once (212 VGPRs, 2 waves per SIMD); bounded it needs 75 and
// spills nothing.
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(6))) void scatter_fp8_held_kernel(
    const u32x4 *__restrict__ x, int64_t T, int64_t chunks, int32_t k,
    const int32_t *__restrict__ src2dst, Fp8Out o, int64_t cap_rows, int32_t *__restrict__ status)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowTok + wave_id();
    if (t >= T) return;
    // lane j < k holds the destination of slot j
    const int32_t dlane = lane < k ? src2dst[t * k + lane] : -1;
    if (__ballot(dlane >= 0) == 0) return;
    const rsrc_t xr = make_rsrc(x + t * chunks, (uint32_t)(chunks * 16));
    u32x4 v[2 * kHeldPairs], q[kHeldPairs];
    uint32_t sw = 0;
    load_fp8_first_parts(v, xr, lane, 0);
    convert_held_row<kRowsFp8>(v, xr, lane, chunks, (o.flags & CDL_FP8_SCALE_UE8M0) != 0, 1.0f, 1.0f,
                               q, sw);
    const bool has = lane < k && dlane >= 0;
    const bool fits = has && (int64_t)dlane < cap_rows;
    if (__ballot(has && !fits) != 0 && lane == 0) set_status(status, CDL_STATUS_ROWS_OVERFLOW);
    store_held_row<true>(q, sw, lane, chunks, o, dlane, __ballot(fits));
}

// Any H, any 2-byte alignment: element-wise copy.
__global__ __launch_bounds__(128) void scatter_rows_u16(
    const uint16_t *__restrict__ x, int64_t H, int32_t k, const int32_t *__restrict__ src2dst,
    uint16_t *__restrict__ out, int64_t cap_rows, int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int32_t *d = src2dst + t * k;
    for (int j = 0; j < k; ++j) {
        const int32_t dst = d[j];
        if (dst < 0) continue;
        if (dst >= cap_rows) {
            if (threadIdx.x == 0) set_status(status, CDL_STATUS_ROWS_OVERFLOW);
            continue;
        }
        for (int64_t h = threadIdx.x; h < H; h += 128) out[(int64_t)dst * H + h] = x[t * H + h];
    }
}

// ---------------------------------------------------------------------------
// rank layout (before the exchange)
// ---------------------------------------------------------------------------

constexpr int kRankThreads = 64;         // tokens per workgroup (one wave), one per thread
constexpr int kRankMaskMax = 64;         // ranks a token's bitmask holds (the fast kernel)

// Per-workgroup partial counts for num_ranks <= 64, one wave per workgroup:
// the token's ids arrive in batches of 8 loads, its ranks and nodes are bit
// masks (a rank or node is counted once per token however many of the
// token's slots it hosts), the per-rank and per-node counts of the wave are
// ballots, and the expert counts an LDS histogram.  Same partial layout as
// below.
__global__ __launch_bounds__(kRankThreads) void rank_layout_mask_kernel(
    const int32_t *__restrict__ ids, int64_t T, int32_t k, int32_t E, int32_t R, int32_t rpn,
    uint8_t *__restrict__ in_rank, int32_t *__restrict__ partial)
{
    extern __shared__ int32_t h[];
    const int N = R / rpn;
    const int W = E + R + N;
    const int lane = threadIdx.x;
    for (int i = lane; i < E; i += kRankThreads) h[i] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * kRankThreads;
    const int64_t t = t0 + lane;
    const bool real = t < T;
    const int32_t epr = E / R;
    // one descriptor for the workgroup's ids (a per-lane one would make the
    // compiler loop over the lanes' descriptors); lane offsets select tokens
    const int64_t ntok = T - t0 < kRankThreads ? T - t0 : kRankThreads;
    const rsrc_t r_ids = make_rsrc(ids + t0 * k, (uint32_t)(ntok * k * 4));
    const uint32_t my_off = (uint32_t)(lane * k) * 4u;
    uint64_t rmask = 0, nmask = 0;
    for (int j0 = 0; j0 < k; j0 += 8) {
        int32_t idv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) idv[q] = buf_ld4(r_ids, my_off + (uint32_t)(j0 + q) * 4u, 0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int32_t id = idv[q];
            if (!real || j0 + q >= k || id < 0 || id >= E) continue;
            atomicAdd(&h[id], 1);
            const int32_t r = id / epr;
            rmask |= 1ull << r;
            nmask |= 1ull << (r / rpn);
        }
    }
    if (real) {
        uint8_t *row = in_rank + t * R;
        if (R % 8 == 0 && ((uintptr_t)in_rank & 7) == 0) {
            // eight flags per 8-byte store
            for (int r0 = 0; r0 < R; r0 += 8) {
                const uint32_t b = (uint32_t)(rmask >> r0) & 0xFFu;
                uint64_t wv = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) wv |= (uint64_t)((b >> i) & 1u) << (8 * i);
                *reinterpret_cast<uint64_t *>(row + r0) = wv;
            }
        } else {
            for (int r = 0; r < R; ++r) row[r] = (uint8_t)((rmask >> r) & 1u);
        }
    }
    // lane r < R ends up with rank r's count, lane n < N with node n's
    int32_t rc = 0, nc = 0;
    for (int r = 0; r < R; ++r) {
        const int32_t c = __popcll(__ballot((rmask >> r) & 1u));
        if (lane == r) rc = c;
    }
    for (int n = 0; n < N; ++n) {
        const int32_t c = __popcll(__ballot((nmask >> n) & 1u));
        if (lane == n) nc = c;
    }
    int32_t *out = partial + (int64_t)blockIdx.x * W;
    if (lane < R) out[E + lane] = rc;
    if (lane < N) out[E + R + lane] = nc;
    __syncthreads();
    for (int i = lane; i < E; i += kRankThreads) out[i] = h[i];
}

// Per-workgroup partial counts: partial[blk][0, E) slots per expert,
// [E, E+R) tokens per rank, [E+R, E+R+N) tokens per node; each token also
// writes its is_token_in_rank row.  A rank (node) counts a token once: only
// the first of the token's valid slots on that rank (node) adds to it.
__global__ __launch_bounds__(kRankThreads) void rank_layout_kernel(
    const int32_t *__restrict__ ids, int64_t T, int32_t k, int32_t E, int32_t R, int32_t rpn,
    uint8_t *__restrict__ in_rank, int32_t *__restrict__ partial)
{
    extern __shared__ int32_t h[];
    const int N = R / rpn;
    const int W = E + R + N;
    for (int i = threadIdx.x; i < W; i += kRankThreads) h[i] = 0;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kRankThreads + threadIdx.x;
    if (t < T) {
        const int32_t epr = E / R;
        const int32_t *my = ids + t * k;
        uint8_t *row = in_rank + t * R;
        for (int r = 0; r < R; ++r) row[r] = 0;
        for (int j = 0; j < k; ++j) {
            const int32_t id = my[j];
            if (id < 0 || id >= E) continue;
            atomicAdd(&h[id], 1);
            const int32_t r = id / epr;
            const int32_t n = r / rpn;
            bool first_r = true, first_n = true;
            for (int j2 = 0; j2 < j; ++j2) {
                const int32_t id2 = my[j2];
                if (id2 < 0 || id2 >= E) continue;
                const int32_t r2 = id2 / epr;
                first_r &= r2 != r;
                first_n &= r2 / rpn != n;
            }
            if (first_r) {
                row[r] = 1;
                atomicAdd(&h[E + r], 1);
            }
            if (first_n) atomicAdd(&h[E + R + n], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < W; i += kRankThreads) partial[(int64_t)blockIdx.x * W + i] = h[i];
}

// Column sums of the partial counts into the three outputs.  A workgroup
// takes 64 columns, and its wave w adds the partial rows w, w + 16, ... with
// 8 loads in flight per batch (one batch per 128 rows: at 4096 tokens the
// 64 rows arrive in one memory round trip instead of 8 dependent ones); wave
// 0 then adds the 16 wave sums from LDS.
constexpr int kRankReduceWaves = 16;
__global__ __launch_bounds__(kRankReduceWaves * kWave) void rank_layout_reduce_kernel(
    const int32_t *__restrict__ partial, int64_t nblocks, int32_t E, int32_t R, int32_t N,
    int32_t *__restrict__ per_expert, int32_t *__restrict__ per_rank, int32_t *__restrict__ per_node)
{
    __shared__ int32_t wsum[kRankReduceWaves][kWave];
    const int W = E + R + N;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int i = blockIdx.x * kWave + lane;
    int32_t sum = 0;
    if (i < W) {
        for (int64_t b = w; b < nblocks; b += 8 * kRankReduceWaves) {
            int32_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t bq = b + (int64_t)q * kRankReduceWaves;
                v[q] = bq < nblocks ? partial[bq * W + i] : 0;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) sum += v[q];
        }
    }
    wsum[w][lane] = sum;
    __syncthreads();
    if (w != 0 || i >= W) return;
#pragma unroll
    for (int q = 1; q < kRankReduceWaves; ++q) sum += wsum[q][lane];
    if (i < E) per_expert[i] = sum;
    else if (i < E + R) per_rank[i - E] = sum;
    else if (per_node) per_node[i - E - R] = sum;
}

// ---------------------------------------------------------------------------
// low-latency dispatch
// ---------------------------------------------------------------------------

// The destination of valid slot i in the padded buffer is row
// e*cap + (src2dst[i] - seg_indptr[e]).
__device__ __forceinline__ int64_t ll_row(const int32_t *__restrict__ ids, int32_t expert_begin,
                                          int32_t L, const int32_t *__restrict__ src2dst,
                                          const int64_t *__restrict__ seg_indptr, int64_t cap,
                                          int64_t i, bool *overflow)
{
    const int32_t d = src2dst[i];
    *overflow = false;
    if (d < 0) return -1;
    const int32_t e = local_expert(ids[i], expert_begin, L);
    if (e < 0) return -1;               // ids disagree with src2dst: drop
    const int64_t slot = (int64_t)d - seg_indptr[e];
    if (slot < 0) return -1;
    if (slot >= cap) {
        *overflow = true;
        return -1;
    }
    return (int64_t)e * cap + slot;
}

// One wave per token (kRowTok per workgroup); workgroups whose index is below
// ceil(L / threads) also write masked_m; waves at or beyond T stop there.
template <bool FP8>
__global__ __launch_bounds__(kRowThreads) void scatter_rows_ll(
    const u32x4 *__restrict__ x, int64_t T, int64_t chunks, int32_t k,
    const int32_t *__restrict__ ids, int32_t expert_begin, int32_t L,
    const int32_t *__restrict__ src2dst, const int64_t *__restrict__ seg_indptr,
    const int32_t *__restrict__ counts, int64_t cap, u32x4 *__restrict__ out, Fp8Out fp8,
    int32_t *__restrict__ masked_m, int32_t *__restrict__ ll_src2dst,
    int32_t *__restrict__ status)
{
    constexpr int NC = FP8 ? kMaxChunksFp8 : kMaxChunks;
    {
        const int64_t e = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
        if (e < L) masked_m[e] = (int32_t)((int64_t)counts[e] < cap ? counts[e] : cap);
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowTok + wave_id();
    if (t >= T) return;
    // lane j < k computes the padded-buffer row of slot j (one dependent load
    // chain for all slots); readlane gives it to the whole wave below
    bool ovf = false;
    const int32_t rlane = lane < k ? (int32_t)ll_row(ids, expert_begin, L, src2dst, seg_indptr, cap,
                                                     t * k + lane, &ovf)
                                   : -1;
    if (lane < k) ll_src2dst[t * k + lane] = rlane;
    if (__ballot(ovf) != 0 && lane == 0) set_status(status, CDL_STATUS_LL_OVERFLOW);
    if (__ballot(rlane >= 0) == 0) return;
    const uint32_t row_bytes = (uint32_t)(chunks * 16);
    const uint32_t voff = (uint32_t)lane * 16u;
    const rsrc_t xr = make_rsrc(x + t * chunks, row_bytes);
    for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)NC * kWave) {
        const uint32_t pass = (uint32_t)(c0 * 16);
        u32x4 v[NC];
        if (FP8) {
            load_fp8_first_parts(v, xr, lane, c0);
        } else {
#pragma unroll
            for (int u = 0; u < NC; ++u) v[u] = buf_ld16(xr, voff, pass + u * kWave * 16);
        }
        if (FP8) {
            const bool ue8m0 = (fp8.flags & CDL_FP8_SCALE_UE8M0) != 0;
            quant_store_pass(v, lane, c0, chunks, fp8, ue8m0, rlane, __ballot(lane < k && rlane >= 0), xr);
            continue;
        }
        for (int j = 0; j < k; ++j) {
            const int64_t row = __builtin_amdgcn_readlane(rlane, j);
            if (row < 0) continue;
            const rsrc_t o = make_rsrc(out + row * chunks, row_bytes);
#pragma unroll
            for (int u = 0; u < NC; ++u) buf_st16(o, v[u], voff, pass + u * kWave * 16);
        }
    }
}

// ---------------------------------------------------------------------------
// combine: gather + weighted fp32 reduce
// ---------------------------------------------------------------------------

// Chunks per lane and slots in flight of the combine.
constexpr int kCombChunks = 2;
constexpr int kCombDepth = 2;
constexpr int kCombMaxThreads = 1024;

// Threads of a combine workgroup: enough lanes for a row at kCombChunks
// chunks each, rounded up to a whole wave (448 at H = 7168; rows longer than
// kCombMaxThreads * kCombChunks chunks take several passes).
inline unsigned comb_threads(int64_t chunks)
{
    const int64_t lanes = (chunks + kCombChunks - 1) / kCombChunks;
    const int64_t t = (lanes + kWave - 1) / kWave * kWave;
    return (unsigned)(t < kCombMaxThreads ? t : kCombMaxThreads);
}

// One workgroup per token, kCombChunks 16-byte chunks per lane, with the rows
// of up to kCombDepth valid slots in flight at once: buffer d holds the d-th
// next valid slot, and each is reloaded with the next valid slot as soon as
// it has been added.  acc = fma(w_j, y_j, acc) over the valid slots j in
// ascending order from +0 (v_fma_f32 is correctly rounded), one bf16
// rounding.  45 VGPRs, so 8 waves per SIMD.  Measured at T = 4096,
// H = 7168, top-8 over 32 of 256 experts, against one slot at a time with
// 7 chunks per lane on 128 threads (105 VGPRs): 20.4 -> 19.6 us inside the
// step, 27.8 -> 25.6 us when the rows come from HBM.  The lanes past the row
// end read and write nothing (buffer range).
__global__ __launch_bounds__(kCombMaxThreads) void combine_rows_pipe(
    const u32x4 *__restrict__ y, int64_t y_rows, int64_t chunks, const int32_t *__restrict__ map,
    const float *__restrict__ wts, int32_t k, u32x4 *__restrict__ out,
    int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int nthr = blockDim.x;
    // lane j < k of each wave holds slot j's row and weight (readlane below:
    // no dependent load per slot); `valid` lists the slots with a row
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t mlane = lane < k ? map[t * k + lane] : -1;
    const float wlane = lane < k ? wts[t * k + lane] : 0.0f;
    const bool bad = lane < k && mlane >= 0 && (int64_t)mlane >= y_rows;
    if (__ballot(bad) != 0 && threadIdx.x == 0) set_status(status, CDL_STATUS_MAP_RANGE);
    const uint64_t valid = __ballot(lane < k && mlane >= 0 && (int64_t)mlane < y_rows);
    const uint32_t row_bytes = (uint32_t)(chunks * 16);
    const uint32_t voff = threadIdx.x * 16u;
    const rsrc_t orow = make_rsrc(out + t * chunks, row_bytes);
    for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)nthr * kCombChunks) {
        const uint32_t pass = (uint32_t)(c0 * 16);
        const uint32_t stride = (uint32_t)nthr * 16u;
        float acc[kCombChunks][8];
#pragma unroll
        for (int u = 0; u < kCombChunks; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
        auto load = [&](int j, u32x4 (&v)[kCombChunks]) {
            const int32_t r = __builtin_amdgcn_readlane(mlane, j);
            const rsrc_t yr = make_rsrc(y + (int64_t)r * chunks, row_bytes);
#pragma unroll
            for (int u = 0; u < kCombChunks; ++u) v[u] = buf_ld16_stream(yr, voff, pass + u * stride);
        };
        auto accum = [&](int j, const u32x4 (&v)[kCombChunks]) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wlane), j));
#pragma unroll
            for (int u = 0; u < kCombChunks; ++u) {
                acc[u][0] = fmaf(wj, bf16_lo(v[u].x), acc[u][0]);
                acc[u][1] = fmaf(wj, bf16_hi(v[u].x), acc[u][1]);
                acc[u][2] = fmaf(wj, bf16_lo(v[u].y), acc[u][2]);
                acc[u][3] = fmaf(wj, bf16_hi(v[u].y), acc[u][3]);
                acc[u][4] = fmaf(wj, bf16_lo(v[u].z), acc[u][4]);
                acc[u][5] = fmaf(wj, bf16_hi(v[u].z), acc[u][5]);
                acc[u][6] = fmaf(wj, bf16_lo(v[u].w), acc[u][6]);
                acc[u][7] = fmaf(wj, bf16_hi(v[u].w), acc[u][7]);
            }
        };
        uint64_t m = valid;
        u32x4 buf[kCombDepth][kCombChunks];
        int js[kCombDepth];
#pragma unroll
        for (int d = 0; d < kCombDepth; ++d) {
            js[d] = -1;
            if (m) {
                js[d] = __builtin_ctzll(m);
                m &= m - 1;
                load(js[d], buf[d]);
            }
        }
        bool more = js[0] >= 0;
        while (more) {
#pragma unroll
            for (int d = 0; d < kCombDepth; ++d) {
                if (more && js[d] >= 0) {
                    accum(js[d], buf[d]);
                    js[d] = -1;
                    if (m) {
                        js[d] = __builtin_ctzll(m);
                        m &= m - 1;
                        load(js[d], buf[d]);
                    }
                } else {
                    more = false;
                }
            }
        }
        // The whole offset goes in the VGPR operand, soffset = 0: the
        // compiler then keeps the next VALU write of the 16-byte store's data
        // registers one wait state away (with an SGPR soffset it reused them
        // at once, and on gfx950 the last four lanes of each 16 then stored
        // the new values now and then: wrong sums in about one token in ten)
#pragma unroll
        for (int u = 0; u < kCombChunks; ++u)
            buf_st16_stream(orow,
                            u32x4{pack_bf16_rne(acc[u][0], acc[u][1]), pack_bf16_rne(acc[u][2], acc[u][3]),
                                  pack_bf16_rne(acc[u][4], acc[u][5]), pack_bf16_rne(acc[u][6], acc[u][7])},
                            voff + pass + u * stride, 0);
    }
}

// Small batches: one workgroup per token and one 16-byte chunk per thread, so
// that the loads of all of a token's slots are in flight together (the
// kernel above reads a token's slots one after another, which sets the time
// of a batch too small to fill the GPU).  Same fma order as above: ascending
// valid slots from +0, one bf16 rounding.  k <= kWideK, y_rows >= 1.
constexpr int kWideK = 8;
constexpr int kWideMaxThreads = 1024;
// batches up to this size use it (measured at H = 7168, top-8: 2.1 us faster
// at 512 tokens, 1.4 us slower at 1024, where the other kernel fills the GPU)
constexpr int64_t kWideMaxTokens = 512;

__global__ __launch_bounds__(kWideMaxThreads) void combine_rows_wide(
    const u32x4 *__restrict__ y, int64_t y_rows, int64_t chunks, const int32_t *__restrict__ map,
    const float *__restrict__ wts, int32_t k, u32x4 *__restrict__ out,
    int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t mlane = lane < k ? map[t * k + lane] : -1;
    const float wlane = lane < k ? wts[t * k + lane] : 0.0f;
    // every slot's row (-1: none) in scalars before any row load, so that no
    // wait for the map falls between the row loads
    int32_t rs[kWideK];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kWideK; ++j) {
        int32_t r = j < k ? __builtin_amdgcn_readlane(mlane, j) : -1;
        if ((int64_t)r >= y_rows) {
            bad = true;
            r = -1;
        }
        rs[j] = r;
    }
    if (bad && threadIdx.x == 0) set_status(status, CDL_STATUS_MAP_RANGE);
    const uint32_t row_bytes = (uint32_t)(chunks * 16);
    const uint32_t voff = threadIdx.x * 16u;
    const rsrc_t orow = make_rsrc(out + t * chunks, row_bytes);
    for (int64_t c0 = 0; c0 < chunks; c0 += blockDim.x) {
        const uint32_t pass = (uint32_t)(c0 * 16);
        // issued for every slot: an unused slot gets an empty range (its loads
        // return 0 and touch no memory), so the wait for slot j's data counts
        // exactly the loads issued after it
        u32x4 v[kWideK];
#pragma unroll
        for (int j = 0; j < kWideK; ++j) {
            const bool use = rs[j] >= 0;
            v[j] = buf_ld16_stream(make_rsrc(y + (use ? (int64_t)rs[j] * chunks : 0), use ? row_bytes : 0u),
                                   voff, pass);
        }
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < kWideK; ++j) {
            if (rs[j] < 0) continue;
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wlane), j));
            acc[0] = fmaf(wj, bf16_lo(v[j].x), acc[0]);
            acc[1] = fmaf(wj, bf16_hi(v[j].x), acc[1]);
            acc[2] = fmaf(wj, bf16_lo(v[j].y), acc[2]);
            acc[3] = fmaf(wj, bf16_hi(v[j].y), acc[3]);
            acc[4] = fmaf(wj, bf16_lo(v[j].z), acc[4]);
            acc[5] = fmaf(wj, bf16_hi(v[j].z), acc[5]);
            acc[6] = fmaf(wj, bf16_lo(v[j].w), acc[6]);
            acc[7] = fmaf(wj, bf16_hi(v[j].w), acc[7]);
        }
        // soffset = 0 (the offset in the VGPR operand), as in
        // combine_rows_pipe: the compiler then spaces the next VALU write of
        // the store's data registers
        buf_st16_stream(orow,
                        u32x4{pack_bf16_rne(acc[0], acc[1]), pack_bf16_rne(acc[2], acc[3]),
                              pack_bf16_rne(acc[4], acc[5]), pack_bf16_rne(acc[6], acc[7])},
                        voff + pass, 0);
    }
}

// Any H, any 2-byte alignment.
__global__ __launch_bounds__(128) void combine_rows_u16(
    const uint16_t *__restrict__ y, int64_t y_rows, int64_t H, const int32_t *__restrict__ map,
    const float *__restrict__ wts, int32_t k, uint16_t *__restrict__ out,
    int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int32_t *m = map + t * k;
    const float *w = wts + t * k;
    for (int64_t h = threadIdx.x; h < H; h += 128) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int32_t r = m[j];
            if (r < 0) continue;
            if ((int64_t)r >= y_rows) {
                if (h == threadIdx.x && threadIdx.x == 0) set_status(status, CDL_STATUS_MAP_RANGE);
                continue;
            }
            acc = fmaf(w[j], __uint_as_float((uint32_t)y[(int64_t)r * H + h] << 16), acc);
        }
        out[t * H + h] = (uint16_t)(pack_bf16_rne(acc, 0.0f) & 0xFFFFu);
    }
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int launch_status()
{
    return hipGetLastError() == hipSuccess ? CDL_OK : CDL_ERR_HIP;
}

inline int check_tk(int64_t T, int32_t k)
{
    if (T < 0 || k < 1 || k > CDL_MAX_TOPK) return CDL_ERR_BAD_SIZE;
    if (T > (int64_t)INT32_MAX / k) return CDL_ERR_TOO_LARGE;
    return CDL_OK;
}

constexpr int kMaxTpbBf16 = 8;
constexpr int kMaxTpbFp8 = 4;

inline size_t layout_ws_bytes(int64_t T, int32_t k, int32_t L)
{
    // one workspace serves every mode: the larger of the two plans
    const int64_t S8 = make_plan(T, k, L, kMaxTpbBf16).S;
    const int64_t S4 = make_plan(T, k, L, kMaxTpbFp8).S;
    const size_t bytes = (size_t)(S8 > S4 ? S8 : S4) * (size_t)L * sizeof(int32_t);
    return ((bytes + 255) & ~(size_t)255) + 256;
}

inline int check_layout_args(const int32_t *topk_ids, int64_t T, int32_t k, int32_t L,
                             int32_t alignment, const int32_t *counts, const int64_t *seg_indptr,
                             const int32_t *src2dst, const int32_t *reorder, int64_t reorder_cap,
                             const void *ws, size_t ws_bytes)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (L < 1 || L > CDL_MAX_LOCAL_EXPERTS) return CDL_ERR_BAD_SIZE;
    if (alignment < 1 || alignment > CDL_MAX_ALIGNMENT || reorder_cap < 0) return CDL_ERR_BAD_SIZE;
    // the largest padded row index must stay below 2^31
    if (T * k + (int64_t)L * (alignment - 1) > (int64_t)INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (!counts || !seg_indptr) return CDL_ERR_NULL_POINTER;
    if (T > 0 && (!topk_ids || !src2dst)) return CDL_ERR_NULL_POINTER;
    if (reorder_cap > 0 && !reorder) return CDL_ERR_NULL_POINTER;
    if (!ws) return CDL_ERR_NULL_POINTER;
    if (ws_bytes < layout_ws_bytes(T, k, L)) return CDL_ERR_WORKSPACE;
    return CDL_OK;
}

inline bool valid_scale_flags(int32_t f)
{
    if (f & ~(CDL_FP8_SCALE_UE8M0 | CDL_FP8_SCALE_COLMAJOR | CDL_FP8_SCALE_PACKED)) return false;
    return !(f & CDL_FP8_SCALE_PACKED) || (f & CDL_FP8_SCALE_UE8M0);
}

inline Fp8Out make_fp8_out(uint8_t *q, void *s, int32_t flags, int64_t H, int64_t rows_per_mat)
{
    Fp8Out o;
    o.q = (u32x2 *)q;
    o.s = (uint8_t *)s;
    o.flags = flags;
    o.groups = H / CDL_FP8_GROUP;
    o.rows_per_mat = rows_per_mat > 0 ? rows_per_mat : 1;
    o.ld = (o.rows_per_mat + 3) / 4 * 4;
    return o;
}

// Bytes of a scale buffer for `rows` rows of H elements in the given format.
inline int64_t scale_bytes(int64_t rows, int64_t H, int32_t flags, int64_t rows_per_mat)
{
    const int64_t G = H / CDL_FP8_GROUP;
    const int64_t words = (flags & CDL_FP8_SCALE_PACKED) ? (G + 3) / 4 : G;
    if (flags & CDL_FP8_SCALE_COLMAJOR) {
        const int64_t rpm = rows_per_mat > 0 ? rows_per_mat : 1;
        const int64_t nmat = (rows + rpm - 1) / rpm;
        return nmat * words * ((rpm + 3) / 4 * 4) * 4;
    }
    return rows * words * 4;
}

// Waves per token.  One, except for fp8 rows of small self-counted batches:
// a row quantised on the way is split over 7 waves of 2 chunks per lane (one
// 7168-wide row in one part), which shortens each wave's load -> quantise ->
// store chain while the GPU has SIMDs to spare (low-latency fp8 dispatch of
// 128 tokens, H = 7168, top-8: 17.0 -> 12.2 us).  Full batches keep one wave
// per token: at 4096 tokens two waves of 7 chunks took the fused fp8 permute
// from 22.9 to 28.6 us (twice the waves, not all of them resident).
template <int MODE, bool ALL_ROWS, int TPB>
constexpr int waves_per_token()
{
    if constexpr ((MODE == kRowsFp8 || MODE == kRowsLLFp8) && ALL_ROWS && TPB <= 2)
        return kFp8WavesSmall;
    else
        return 1;
}

template <int MODE, bool ALL_ROWS, int TPB>
void launch_permute_wpt(const PermuteArgs &a, dim3 grid, size_t lds, hipStream_t s)
{
    constexpr int WPT = waves_per_token<MODE, ALL_ROWS, TPB>();
    permute_kernel<TPB, MODE, ALL_ROWS, WPT><<<grid, dim3(TPB * WPT * kWave), lds, s>>>(a);
}

template <int MODE, bool ALL_ROWS>
void launch_permute_tpb(const PermuteArgs &a, const Plan &p, hipStream_t s)
{
    const size_t lds = (size_t)(2 * a.L + p.tpb * a.k) * sizeof(int32_t);
    const dim3 grid((unsigned)(p.nblocks > 0 ? p.nblocks : 1));
    switch (p.tpb) {
    case 1: launch_permute_wpt<MODE, ALL_ROWS, 1>(a, grid, lds, s); break;
    case 2: launch_permute_wpt<MODE, ALL_ROWS, 2>(a, grid, lds, s); break;
    case 4: launch_permute_wpt<MODE, ALL_ROWS, 4>(a, grid, lds, s); break;
    default: launch_permute_wpt<MODE, ALL_ROWS, 8>(a, grid, lds, s); break;
    }
}

// Batches of at most this many tokens that count themselves load every row
// rather than first checking each token for a local slot: at most this many
// rows read in vain (7.3 MB at H = 7168) against one id-load latency saved
// per wave (measured at top-8: 1.0 us faster at 32-128 tokens, 0.4-0.9 us at
// 256-512).
constexpr int64_t kAllRowsMaxTokens = 512;

// The layout alone for batches with superblock counts: one wave per
// workgroup of p.tpb tokens.
inline void launch_layout_wave(const PermuteArgs &a, const Plan &p, hipStream_t s)
{
    const size_t lds = (size_t)(2 * a.L) * sizeof(int32_t);
    const dim3 grid((unsigned)(p.nblocks > 0 ? p.nblocks : 1));
    switch (p.tpb) {
    case 1: layout_wave_kernel<1><<<grid, dim3(kWave), lds, s>>>(a); break;
    case 2: layout_wave_kernel<2><<<grid, dim3(kWave), lds, s>>>(a); break;
    case 4: layout_wave_kernel<4><<<grid, dim3(kWave), lds, s>>>(a); break;
    default: layout_wave_kernel<8><<<grid, dim3(kWave), lds, s>>>(a); break;
    }
}

// fp8 rows of one pass with superblock counts: a layout wave beside the
// row waves (permute_fp8_split_kernel)
template <int MODE>
void launch_fp8_split(const PermuteArgs &a, const Plan &p, hipStream_t s)
{
    const size_t lds = (size_t)(2 * a.L + p.tpb * a.k) * sizeof(int32_t);
    const dim3 grid((unsigned)(p.nblocks > 0 ? p.nblocks : 1));
    switch (p.tpb) {
    case 1: permute_fp8_split_kernel<1, MODE><<<grid, dim3(2 * kWave), lds, s>>>(a); break;
    case 2: permute_fp8_split_kernel<2, MODE><<<grid, dim3(3 * kWave), lds, s>>>(a); break;
    default: permute_fp8_split_kernel<4, MODE><<<grid, dim3(5 * kWave), lds, s>>>(a); break;
    }
}

template <int MODE>
int launch_permute(PermuteArgs a, const Plan &p, hipStream_t s)
{
    if constexpr (MODE == kRowsFp8 || MODE == kRowsFp8Tensor || MODE == kRowsFp8Cast1) {
        // rows of one pass held as whole pairs of chunks (H % 128 == 0 for
        // groups; the per-tensor cast takes any H % 8 == 0, and a row of an
        // odd number of chunks keeps the one-chunk path: a 16-byte store must
        // not straddle the row end)
        if (!a.self_count && a.chunks <= (int64_t)kMaxChunksFp8 * kWave && a.chunks % 2 == 0) {
            launch_fp8_split<MODE>(a, p, s);
            return launch_status();
        }
    }
    if constexpr (MODE == kLayoutOnly) {
        if (a.self_count)
            launch_permute_tpb<MODE, false>(a, p, s);
        else
            launch_layout_wave(a, p, s);
    } else if (a.self_count && a.T > 0 && a.T <= kAllRowsMaxTokens) {
        launch_permute_tpb<MODE, true>(a, p, s);
    } else {
        launch_permute_tpb<MODE, false>(a, p, s);
    }
    return launch_status();
}

// Kernel A (unless the batch counts itself) then kernel B in the given mode.
template <int MODE>
int run_layout(PermuteArgs a, void *ws, hipStream_t s)
{
    // fp8 rows (the split kernel takes up to 4 tokens per workgroup)
    constexpr bool kFp8Rows = MODE == kRowsFp8 || MODE == kRowsLLFp8 || MODE == kRowsFp8Tensor ||
                              MODE == kRowsFp8Cast1;
    const Plan p = make_plan(a.T, a.k, a.L, kFp8Rows ? kMaxTpbFp8 : kMaxTpbBf16);
    a.sb_counts = (const int32_t *)ws;
    a.S = p.S;
    a.sbb_shift = 0;
    while ((int64_t)1 << a.sbb_shift < p.sbb) ++a.sbb_shift;     // sbb is a power of two
    a.sb_slots = p.sb_slots;
    // the superblock-count entries are indexed in 32 bits
    if (p.S * (int64_t)a.L > (int64_t)INT32_MAX) return CDL_ERR_TOO_LARGE;
    // a batch of at most kSelfCountIds ids per thread of a permute workgroup
    // is counted by every workgroup itself, without the count kernel
    a.self_count = p.n <= (int64_t)kSelfCountIds * kWave * p.tpb ? 1 : 0;
    if (p.S > 0 && !a.self_count) {
        layout_count_kernel<<<dim3((unsigned)p.S), dim3(kCountThreads), a.L * sizeof(int32_t), s>>>(
            a.ids, p.n, p.sb_slots, a.expert_begin, a.L, (int32_t *)ws);
        int rc = launch_status();
        if (rc != CDL_OK) return rc;
    }
    return launch_permute<MODE>(a, p, s);
}

PermuteArgs layout_args(const int32_t *topk_ids, int64_t T, int32_t k, int32_t expert_begin,
                        int32_t L, int32_t alignment, int32_t *counts, int64_t *seg_indptr,
                        int32_t *src2dst, int32_t *reorder, int64_t reorder_cap, int32_t *status)
{
    PermuteArgs a = {};
    a.ids = topk_ids;
    a.T = T;
    a.k = k;
    a.expert_begin = expert_begin;
    a.L = L;
    a.alignment = alignment;
    a.counts = counts;
    a.seg_indptr = seg_indptr;
    a.src2dst = src2dst;
    a.reorder = reorder;
    a.reorder_cap = reorder_cap;
    a.status = status;
    return a;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

size_t cdl_dispatch_layout_workspace_size(int64_t T, int32_t k, int32_t L)
{
    if (check_tk(T, k) != CDL_OK || L < 1 || L > CDL_MAX_LOCAL_EXPERTS) return 0;
    return layout_ws_bytes(T, k, L);
}

int cdl_dispatch_layout(const int32_t *topk_ids, int64_t T, int32_t k, int32_t expert_begin,
                        int32_t L, int32_t *counts, int64_t *seg_indptr, int32_t *src2dst,
                        int32_t *reorder_topk_ids, void *ws, size_t ws_bytes, void *stream)
{
    return cdl_dispatch_layout_aligned(topk_ids, T, k, expert_begin, L, 1, counts, seg_indptr,
                                       src2dst, reorder_topk_ids, T * k, nullptr, ws, ws_bytes,
                                       stream);
}

int cdl_dispatch_layout_aligned(const int32_t *topk_ids, int64_t T, int32_t k,
                                int32_t expert_begin, int32_t L, int32_t alignment,
                                int32_t *counts, int64_t *seg_indptr, int32_t *src2dst,
                                int32_t *reorder_topk_ids, int64_t reorder_cap, int32_t *status,
                                void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_layout_args(topk_ids, T, k, L, alignment, counts, seg_indptr, src2dst,
                               reorder_topk_ids, reorder_cap, ws, ws_bytes);
    if (rc != CDL_OK) return rc;
    PermuteArgs a = layout_args(topk_ids, T, k, expert_begin, L, alignment, counts, seg_indptr,
                                src2dst, reorder_topk_ids, reorder_cap, status);
    return run_layout<kLayoutOnly>(a, ws, (hipStream_t)stream);
}

int cdl_permute(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                int32_t expert_begin, int32_t L, int32_t alignment, int32_t *counts,
                int64_t *seg_indptr, int32_t *src2dst, int32_t *reorder_topk_ids,
                int64_t reorder_cap, uint16_t *out, int64_t cap_rows, int32_t *status, void *ws,
                size_t ws_bytes, void *stream)
{
    int rc = check_layout_args(topk_ids, T, k, L, alignment, counts, seg_indptr, src2dst,
                               reorder_topk_ids, reorder_cap, ws, ws_bytes);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap_rows < 0) return CDL_ERR_BAD_SIZE;
    if (H > CDL_MAX_HIDDEN) return CDL_ERR_TOO_LARGE;
    if (cap_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (T > 0 && !x) return CDL_ERR_NULL_POINTER;
    if (cap_rows > 0 && !out) return CDL_ERR_NULL_POINTER;
    if (H % 8 != 0 || !aligned(x, 16) || !aligned(out, 16)) return CDL_ERR_UNSUPPORTED;
    PermuteArgs a = layout_args(topk_ids, T, k, expert_begin, L, alignment, counts, seg_indptr,
                                src2dst, reorder_topk_ids, reorder_cap, status);
    a.x = (const u32x4 *)x;
    a.chunks = H / 8;
    a.out = (u32x4 *)out;
    a.cap_rows = cap_rows;
    return run_layout<kRowsBf16>(a, ws, (hipStream_t)stream);
}

}  // extern "C"

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch[kMaxScratchDevices];     // device address per device
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up (with that device
// current) on the first call there.
int scratch_address(hipStream_t s, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CDL_ERR_HIP;
    if (dev >= kMaxScratchDevices) return CDL_ERR_UNSUPPORTED;
    if (s) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return CDL_ERR_HIP;
        if (sdev != dev) return CDL_ERR_UNSUPPORTED;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CDL_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return CDL_OK;
}

}  // namespace

extern "C" {

int cdl_permute_noalloc(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                        const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                        int32_t alignment, int32_t *counts, int64_t *seg_indptr, int32_t *src2dst,
                        int32_t *reorder_topk_ids, int64_t reorder_cap, uint16_t *out,
                        int64_t cap_rows, int32_t *status, void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (L < 1 || L > CDL_MAX_LOCAL_EXPERTS) return CDL_ERR_BAD_SIZE;
    const size_t need = layout_ws_bytes(T, k, L);
    if (need > (size_t)CDL_NOALLOC_SCRATCH_BYTES) return CDL_ERR_SCRATCH;
    void *ws = nullptr;
    rc = scratch_address((hipStream_t)stream, &ws);
    if (rc != CDL_OK) return rc;
    return cdl_permute(x, T, H, k, topk_ids, expert_begin, L, alignment, counts, seg_indptr,
                       src2dst, reorder_topk_ids, reorder_cap, out, cap_rows, status, ws,
                       (size_t)CDL_NOALLOC_SCRATCH_BYTES, stream);
}

int cdl_permute_fp8_tensor(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                           const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                           int32_t alignment, int32_t *counts, int64_t *seg_indptr,
                           int32_t *src2dst, int32_t *reorder_topk_ids, int64_t reorder_cap,
                           uint8_t *out_q, const float *scale, int64_t cap_rows, int32_t *status,
                           void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_layout_args(topk_ids, T, k, L, alignment, counts, seg_indptr, src2dst,
                               reorder_topk_ids, reorder_cap, ws, ws_bytes);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap_rows < 0) return CDL_ERR_BAD_SIZE;
    if (H > CDL_MAX_HIDDEN) return CDL_ERR_TOO_LARGE;
    if (cap_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (T > 0 && !x) return CDL_ERR_NULL_POINTER;
    if (cap_rows > 0 && !out_q) return CDL_ERR_NULL_POINTER;
    if (H % 8 != 0 || !aligned(x, 16) || !aligned(out_q, 8) || !aligned(scale, 4))
        return CDL_ERR_UNSUPPORTED;
    PermuteArgs a = layout_args(topk_ids, T, k, expert_begin, L, alignment, counts, seg_indptr,
                                src2dst, reorder_topk_ids, reorder_cap, status);
    a.x = (const u32x4 *)x;
    a.chunks = H / 8;
    a.cap_rows = cap_rows;
    a.fp8.q = (u32x2 *)out_q;
    a.tensor_scale = scale;
    if (!scale) return run_layout<kRowsFp8Cast1>(a, ws, (hipStream_t)stream);
    return run_layout<kRowsFp8Tensor>(a, ws, (hipStream_t)stream);
}

size_t cdl_fp8_scale_bytes(int64_t rows, int64_t H, int32_t scale_flags, int64_t rows_per_mat)
{
    if (rows < 0 || H < CDL_FP8_GROUP || H % CDL_FP8_GROUP != 0 || !valid_scale_flags(scale_flags))
        return 0;
    if ((scale_flags & CDL_FP8_SCALE_COLMAJOR) && rows_per_mat < 1) return 0;
    return (size_t)scale_bytes(rows, H, scale_flags, rows_per_mat);
}

size_t cdl_permute_fp8_workspace_size(int64_t T, int32_t k, int32_t L, int64_t H,
                                      int32_t scale_flags, int64_t rows)
{
    if (check_tk(T, k) != CDL_OK || L < 1 || L > CDL_MAX_LOCAL_EXPERTS) return 0;
    if (H < CDL_FP8_GROUP || H > CDL_MAX_HIDDEN || H % CDL_FP8_GROUP != 0 || rows < 0) return 0;
    if (!valid_scale_flags(scale_flags)) return 0;
    return layout_ws_bytes(T, k, L);
}

int cdl_permute_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                    int32_t expert_begin, int32_t L, int32_t alignment, int32_t *counts,
                    int64_t *seg_indptr, int32_t *src2dst, int32_t *reorder_topk_ids,
                    int64_t reorder_cap, uint8_t *out_q, void *out_scales, int32_t scale_flags,
                    int64_t cap_rows, int32_t *status, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_layout_args(topk_ids, T, k, L, alignment, counts, seg_indptr, src2dst,
                               reorder_topk_ids, reorder_cap, ws, ws_bytes);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap_rows < 0) return CDL_ERR_BAD_SIZE;
    if (H > CDL_MAX_HIDDEN) return CDL_ERR_TOO_LARGE;
    if (H % CDL_FP8_GROUP != 0 || !valid_scale_flags(scale_flags)) return CDL_ERR_UNSUPPORTED;
    if (cap_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (T > 0 && !x) return CDL_ERR_NULL_POINTER;
    if (cap_rows > 0 && (!out_q || !out_scales)) return CDL_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(out_q, 8) || !aligned(out_scales, 4)) return CDL_ERR_UNSUPPORTED;
    PermuteArgs a = layout_args(topk_ids, T, k, expert_begin, L, alignment, counts, seg_indptr,
                                src2dst, reorder_topk_ids, reorder_cap, status);
    a.x = (const u32x4 *)x;
    a.chunks = H / 8;
    a.cap_rows = cap_rows;
    a.fp8 = make_fp8_out(out_q, out_scales, scale_flags, H, cap_rows);
    return run_layout<kRowsFp8>(a, ws, (hipStream_t)stream);
}

static int check_rank_layout_sizes(int64_t T, int32_t k, int32_t E, int32_t R, int32_t rpn)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (E < 1 || E > CDL_MAX_EXPERTS || R < 1 || R > CDL_MAX_RANKS || rpn < 1) return CDL_ERR_BAD_SIZE;
    if (E % R != 0 || R % rpn != 0) return CDL_ERR_UNSUPPORTED;
    if (T * R > (int64_t)INT32_MAX) return CDL_ERR_TOO_LARGE;
    return CDL_OK;
}

size_t cdl_rank_layout_workspace_size(int64_t T, int32_t k, int32_t E, int32_t num_ranks,
                                      int32_t ranks_per_node)
{
    if (check_rank_layout_sizes(T, k, E, num_ranks, ranks_per_node) != CDL_OK) return 0;
    const int64_t nblocks = (T + kRankThreads - 1) / kRankThreads;
    const int64_t W = (int64_t)E + num_ranks + num_ranks / ranks_per_node;
    return (size_t)(nblocks * W * 4 + 256);
}

int cdl_rank_layout(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E, int32_t num_ranks,
                    int32_t ranks_per_node, int32_t *num_tokens_per_rank,
                    int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                    uint8_t *is_token_in_rank, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_rank_layout_sizes(T, k, E, num_ranks, ranks_per_node);
    if (rc != CDL_OK) return rc;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !ws) return CDL_ERR_NULL_POINTER;
    if (T > 0 && (!topk_ids || !is_token_in_rank)) return CDL_ERR_NULL_POINTER;
    if (ws_bytes < cdl_rank_layout_workspace_size(T, k, E, num_ranks, ranks_per_node))
        return CDL_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int64_t nblocks = (T + kRankThreads - 1) / kRankThreads;
    const int32_t N = num_ranks / ranks_per_node;
    const int32_t W = E + num_ranks + N;
    if (nblocks > 0) {
        if (num_ranks <= kRankMaskMax)
            rank_layout_mask_kernel<<<dim3((unsigned)nblocks), dim3(kRankThreads), (size_t)E * 4, s>>>(
                topk_ids, T, k, E, num_ranks, ranks_per_node, is_token_in_rank, (int32_t *)ws);
        else
            rank_layout_kernel<<<dim3((unsigned)nblocks), dim3(kRankThreads), (size_t)W * 4, s>>>(
                topk_ids, T, k, E, num_ranks, ranks_per_node, is_token_in_rank, (int32_t *)ws);
        if ((rc = launch_status()) != CDL_OK) return rc;
    }
    rank_layout_reduce_kernel<<<dim3((unsigned)((W + kWave - 1) / kWave)), dim3(kRankReduceWaves * kWave), 0, s>>>(
        (const int32_t *)ws, nblocks, E, num_ranks, N, num_tokens_per_expert, num_tokens_per_rank,
        num_tokens_per_rdma_rank);
    return launch_status();
}

int cdl_dispatch(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *src2dst,
                 uint16_t *out, int64_t cap_rows, int32_t *status, void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap_rows < 0) return CDL_ERR_BAD_SIZE;
    if (H > CDL_MAX_HIDDEN) return CDL_ERR_TOO_LARGE;
    if (T == 0) return CDL_OK;
    if (!x || !src2dst) return CDL_ERR_NULL_POINTER;
    if (cap_rows > 0 && !out) return CDL_ERR_NULL_POINTER;
    if (cap_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    hipStream_t s = (hipStream_t)stream;
    if (H % 8 == 0 && aligned(x, 16) && aligned(out, 16)) {
        scatter_rows_kernel<false><<<dim3((unsigned)((T + kRowTok - 1) / kRowTok)), dim3(kRowThreads), 0, s>>>(
            (const u32x4 *)x, T, H / 8, k, src2dst, (u32x4 *)out, Fp8Out{}, cap_rows, status);
    } else {
        scatter_rows_u16<<<dim3((unsigned)T), dim3(128), 0, s>>>(x, H, k, src2dst, out, cap_rows,
                                                                  status);
    }
    return launch_status();
}

int cdl_dispatch_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *src2dst,
                     uint8_t *out_q, float *out_scales, int64_t cap_rows, int32_t *status,
                     void *stream)
{
    return cdl_dispatch_fp8_ex(x, T, H, k, src2dst, out_q, out_scales, 0, cap_rows, status,
                               stream);
}

int cdl_dispatch_fp8_ex(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                        const int32_t *src2dst, uint8_t *out_q, void *out_scales,
                        int32_t scale_flags, int64_t cap_rows, int32_t *status, void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap_rows < 0) return CDL_ERR_BAD_SIZE;
    if (H > CDL_MAX_HIDDEN) return CDL_ERR_TOO_LARGE;
    if (H % CDL_FP8_GROUP != 0 || !valid_scale_flags(scale_flags)) return CDL_ERR_UNSUPPORTED;
    if (T == 0) return CDL_OK;
    if (!x || !src2dst) return CDL_ERR_NULL_POINTER;
    if (cap_rows > 0 && (!out_q || !out_scales)) return CDL_ERR_NULL_POINTER;
    if (cap_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (!aligned(x, 16) || (cap_rows > 0 && !aligned(out_q, 8)) ||
        (cap_rows > 0 && !aligned(out_scales, 4)))
        return CDL_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)((T + kRowTok - 1) / kRowTok));
    if (H / 8 <= (int64_t)kHeldPairs * 2 * kWave)      // rows of one pass
        scatter_fp8_held_kernel<<<grid, dim3(kRowThreads), 0, s>>>(
            (const u32x4 *)x, T, H / 8, k, src2dst,
            make_fp8_out(out_q, out_scales, scale_flags, H, cap_rows), cap_rows, status);
    else
        scatter_rows_kernel<true><<<grid, dim3(kRowThreads), 0, s>>>(
            (const u32x4 *)x, T, H / 8, k, src2dst, nullptr,
            make_fp8_out(out_q, out_scales, scale_flags, H, cap_rows), cap_rows, status);
    return launch_status();
}

static int check_ll_args(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                         const int32_t *topk_ids, int32_t L, const int32_t *src2dst,
                         const int64_t *seg_indptr, const int32_t *counts, int64_t cap,
                         const void *out, int32_t *masked_m, int32_t *ll_src2dst)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap < 0 || L < 1 || L > CDL_MAX_LOCAL_EXPERTS) return CDL_ERR_BAD_SIZE;
    if (H > CDL_MAX_HIDDEN) return CDL_ERR_TOO_LARGE;
    if (H % 8 != 0) return CDL_ERR_UNSUPPORTED;
    if ((int64_t)L * cap > INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (!counts || !seg_indptr || !masked_m) return CDL_ERR_NULL_POINTER;
    if (T > 0 && (!x || !topk_ids || !src2dst || !ll_src2dst)) return CDL_ERR_NULL_POINTER;
    if (cap > 0 && !out) return CDL_ERR_NULL_POINTER;
    if (T > 0 && !aligned(x, 16)) return CDL_ERR_UNSUPPORTED;
    return CDL_OK;
}

// Layout and low-latency scatter in one call.
static int permute_ll_common(PermuteArgs &a, const uint16_t *x, int64_t T, int64_t H, int32_t k,
                             const int32_t *topk_ids, int32_t L, int32_t *counts,
                             int64_t *seg_indptr, int32_t *src2dst, int32_t *reorder_topk_ids,
                             int64_t reorder_cap, int64_t cap, const void *out, int32_t *masked_m,
                             int32_t *ll_src2dst, const void *ws, size_t ws_bytes)
{
    int rc = check_layout_args(topk_ids, T, k, L, 1, counts, seg_indptr, src2dst, reorder_topk_ids,
                               reorder_cap, ws, ws_bytes);
    if (rc != CDL_OK) return rc;
    rc = check_ll_args(x, T, H, k, topk_ids, L, src2dst, seg_indptr, counts, cap, out, masked_m,
                       ll_src2dst);
    if (rc != CDL_OK) return rc;
    a.x = (const u32x4 *)x;
    a.chunks = H / 8;
    a.cap_rows = (int64_t)L * cap;
    a.ll_cap = cap;
    a.masked_m = masked_m;
    a.ll_src2dst = ll_src2dst;
    return CDL_OK;
}

int cdl_permute_ll(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                   int32_t expert_begin, int32_t L, int32_t *counts, int64_t *seg_indptr,
                   int32_t *src2dst, int32_t *reorder_topk_ids, int64_t reorder_cap, int64_t cap,
                   uint16_t *out, int32_t *masked_m, int32_t *ll_src2dst, int32_t *status, void *ws,
                   size_t ws_bytes, void *stream)
{
    PermuteArgs a = layout_args(topk_ids, T, k, expert_begin, L, 1, counts, seg_indptr, src2dst,
                                reorder_topk_ids, reorder_cap, status);
    int rc = permute_ll_common(a, x, T, H, k, topk_ids, L, counts, seg_indptr, src2dst,
                               reorder_topk_ids, reorder_cap, cap, out, masked_m, ll_src2dst, ws,
                               ws_bytes);
    if (rc != CDL_OK) return rc;
    if (cap > 0 && !aligned(out, 16)) return CDL_ERR_UNSUPPORTED;
    a.out = (u32x4 *)out;
    return run_layout<kRowsLL>(a, ws, (hipStream_t)stream);
}

int cdl_permute_ll_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                       const int32_t *topk_ids, int32_t expert_begin, int32_t L, int32_t *counts,
                       int64_t *seg_indptr, int32_t *src2dst, int32_t *reorder_topk_ids,
                       int64_t reorder_cap, int64_t cap, uint8_t *out_q, void *out_scales,
                       int32_t scale_flags, int32_t *masked_m, int32_t *ll_src2dst,
                       int32_t *status, void *ws, size_t ws_bytes, void *stream)
{
    PermuteArgs a = layout_args(topk_ids, T, k, expert_begin, L, 1, counts, seg_indptr, src2dst,
                                reorder_topk_ids, reorder_cap, status);
    int rc = permute_ll_common(a, x, T, H, k, topk_ids, L, counts, seg_indptr, src2dst,
                               reorder_topk_ids, reorder_cap, cap, out_q, masked_m, ll_src2dst, ws,
                               ws_bytes);
    if (rc != CDL_OK) return rc;
    if (H % CDL_FP8_GROUP != 0 || !valid_scale_flags(scale_flags)) return CDL_ERR_UNSUPPORTED;
    if (cap > 0 && !out_scales) return CDL_ERR_NULL_POINTER;
    if (cap > 0 && (!aligned(out_q, 8) || !aligned(out_scales, 4))) return CDL_ERR_UNSUPPORTED;
    a.fp8 = make_fp8_out(out_q, out_scales, scale_flags, H, cap);
    return run_layout<kRowsLLFp8>(a, ws, (hipStream_t)stream);
}


// one wave per token; at least enough workgroups to write masked_m
static dim3 ll_grid(int64_t T, int32_t L)
{
    const int64_t mm_blocks = (L + kRowThreads - 1) / kRowThreads;
    const int64_t tok_blocks = (T + kRowTok - 1) / kRowTok;
    return dim3((unsigned)(tok_blocks > mm_blocks ? tok_blocks : mm_blocks));
}

int cdl_dispatch_ll(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                    int32_t expert_begin, int32_t L, const int32_t *src2dst,
                    const int64_t *seg_indptr, const int32_t *counts, int64_t cap, uint16_t *out,
                    int32_t *masked_m, int32_t *ll_src2dst, int32_t *status, void *stream)
{
    int rc = check_ll_args(x, T, H, k, topk_ids, L, src2dst, seg_indptr, counts, cap, out,
                           masked_m, ll_src2dst);
    if (rc != CDL_OK) return rc;
    if (cap > 0 && !aligned(out, 16)) return CDL_ERR_UNSUPPORTED;
    scatter_rows_ll<false><<<ll_grid(T, L), dim3(kRowThreads), 0, (hipStream_t)stream>>>(
        (const u32x4 *)x, T, H / 8, k, topk_ids, expert_begin, L, src2dst, seg_indptr, counts,
        cap, (u32x4 *)out, Fp8Out{}, masked_m, ll_src2dst, status);
    return launch_status();
}

int cdl_dispatch_ll_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                        const int32_t *topk_ids, int32_t expert_begin, int32_t L,
                        const int32_t *src2dst, const int64_t *seg_indptr, const int32_t *counts,
                        int64_t cap, uint8_t *out_q, void *out_scales, int32_t scale_flags,
                        int32_t *masked_m, int32_t *ll_src2dst, int32_t *status, void *stream)
{
    int rc = check_ll_args(x, T, H, k, topk_ids, L, src2dst, seg_indptr, counts, cap, out_q,
                           masked_m, ll_src2dst);
    if (rc != CDL_OK) return rc;
    if (H % CDL_FP8_GROUP != 0 || !valid_scale_flags(scale_flags)) return CDL_ERR_UNSUPPORTED;
    if (cap > 0 && !out_scales) return CDL_ERR_NULL_POINTER;
    if (cap > 0 && (!aligned(out_q, 8) || !aligned(out_scales, 4))) return CDL_ERR_UNSUPPORTED;
    scatter_rows_ll<true><<<ll_grid(T, L), dim3(kRowThreads), 0, (hipStream_t)stream>>>(
        (const u32x4 *)x, T, H / 8, k, topk_ids, expert_begin, L, src2dst, seg_indptr, counts,
        cap, nullptr, make_fp8_out(out_q, out_scales, scale_flags, H, cap), masked_m, ll_src2dst,
        status);
    return launch_status();
}

static int run_combine(const uint16_t *y, int64_t y_rows, int64_t H, const int32_t *map,
                       const float *topk_weights, int64_t T, int32_t k, uint16_t *out,
                       int32_t *status, hipEvent_t start, hipEvent_t stop, void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || y_rows < 0) return CDL_ERR_BAD_SIZE;
    if (H > CDL_MAX_HIDDEN) return CDL_ERR_TOO_LARGE;
    if (T == 0) return CDL_OK;
    if (!map || !topk_weights || !out) return CDL_ERR_NULL_POINTER;
    if (y_rows > 0 && !y) return CDL_ERR_NULL_POINTER;
    if (y_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    hipStream_t s = (hipStream_t)stream;
    const bool timed = start != nullptr || stop != nullptr;
    if (H % 8 == 0 && aligned(y, 16) && aligned(out, 16) && k <= kWideK && T <= kWideMaxTokens &&
        y_rows > 0) {
        const int64_t chunks = H / 8;
        const unsigned nt = (unsigned)(chunks >= kWideMaxThreads ? kWideMaxThreads : (chunks + kWave - 1) / kWave * kWave);
        if (timed)
            hipExtLaunchKernelGGL(combine_rows_wide, dim3((unsigned)T), dim3(nt), 0, s, start, stop, 0,
                                  (const u32x4 *)y, y_rows, chunks, map, topk_weights, k,
                                  (u32x4 *)out, status);
        else
            combine_rows_wide<<<dim3((unsigned)T), dim3(nt), 0, s>>>(
                (const u32x4 *)y, y_rows, chunks, map, topk_weights, k, (u32x4 *)out, status);
    } else if (H % 8 == 0 && aligned(y, 16) && aligned(out, 16)) {
        const dim3 block(comb_threads(H / 8));
        if (timed)   // the launch itself carries the events
            hipExtLaunchKernelGGL(combine_rows_pipe, dim3((unsigned)T), block, 0, s, start, stop, 0,
                                  (const u32x4 *)y, y_rows, H / 8, map, topk_weights, k,
                                  (u32x4 *)out, status);
        else
            combine_rows_pipe<<<dim3((unsigned)T), block, 0, s>>>(
                (const u32x4 *)y, y_rows, H / 8, map, topk_weights, k, (u32x4 *)out, status);
    } else {
        if (timed)
            hipExtLaunchKernelGGL(combine_rows_u16, dim3((unsigned)T), dim3(128), 0, s, start, stop, 0,
                                  y, y_rows, H, map, topk_weights, k, out, status);
        else
            combine_rows_u16<<<dim3((unsigned)T), dim3(128), 0, s>>>(y, y_rows, H, map, topk_weights,
                                                                      k, out, status);
    }
    return launch_status();
}

int cdl_combine(const uint16_t *y, int64_t y_rows, int64_t H, const int32_t *map,
                const float *topk_weights, int64_t T, int32_t k, uint16_t *out, int32_t *status,
                void *stream)
{
    return run_combine(y, y_rows, H, map, topk_weights, T, k, out, status, nullptr, nullptr, stream);
}

int cdl_combine_timed(const uint16_t *y, int64_t y_rows, int64_t H, const int32_t *map,
                      const float *topk_weights, int64_t T, int32_t k, uint16_t *out,
                      int32_t *status, void *start_event, void *stop_event, void *stream)
{
    return run_combine(y, y_rows, H, map, topk_weights, T, k, out, status, (hipEvent_t)start_event,
                       (hipEvent_t)stop_event, stream);
}

int64_t cdl_ll_expected_m(int64_t T, int32_t num_ranks, int32_t k, int32_t E)
{
    if (E <= 0 || T < 0 || num_ranks < 0 || k < 0) return -1;
    return (T * (int64_t)num_ranks * (int64_t)k + (int64_t)E) / (int64_t)E;
}

const char *cdl_status_string(int code)
{
    switch (code) {
    case CDL_OK: return "ok";
    case CDL_ERR_NULL_POINTER: return "a required pointer is NULL";
    case CDL_ERR_BAD_SIZE: return "size out of range (T, H, k, L or capacity)";
    case CDL_ERR_UNSUPPORTED: return "unsupported shape or alignment for this operation";
    case CDL_ERR_WORKSPACE: return "workspace smaller than required";
    case CDL_ERR_TOO_LARGE: return "sizes need 2^31 or more slots or rows";
    case CDL_ERR_HIP: return "HIP kernel launch failed";
    case CDL_ERR_SCRATCH: return "the call needs more scratch than the static buffer of cdl_permute_noalloc holds";
    default: return "unknown cdl status code";
    }
}

}  // extern "C"
