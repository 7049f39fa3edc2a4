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
//   * 64-lane wavefronts: the layout ranks slots with wave ballots
//     (__ballot / popcount / readlane) instead of atomics, so src2dst is
//     deterministic and stable by flat slot index.
//   * Row kernels move 16 bytes per lane per access (global_load_dwordx4 /
//     global_store_dwordx4) and keep all of a lane's chunks of a row in
//     registers, so each source row is read once whatever its fan-out.
//   * Routing indices are block-uniform and land in scalar registers.
//   * No kernel keeps state across calls; nothing needs zeroing except the
//     caller's status word.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cdl.h"

namespace {

constexpr int kWave = 64;

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
// layout: per-tile histogram, then scan + stable rank
// ---------------------------------------------------------------------------

constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / kWave;          // 4
constexpr int kTile = 1024;                                   // slots per tile
constexpr int kSlotsPerWave = kTile / kLayoutWaves;            // 256
constexpr int kGroupsPerWave = kSlotsPerWave / kWave;          // 4

inline int64_t layout_tiles(int64_t n) { return (n + kTile - 1) / kTile; }

// Kernel 1: tile_counts[tile][e] = number of valid slots of expert e in the
// tile (an LDS histogram; the count is order independent).
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int32_t *__restrict__ ids, int64_t n, int32_t expert_begin, int32_t L,
    int32_t *__restrict__ tile_counts)
{
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < L; e += kLayoutThreads) hist[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kTile;
    for (int s = threadIdx.x; s < kTile; s += kLayoutThreads) {
        const int64_t i = base + s;
        if (i < n) {
            const int32_t e = local_expert(ids[i], expert_begin, L);
            if (e >= 0) atomicAdd(&hist[e], 1);
        }
    }
    __syncthreads();
    int32_t *row = tile_counts + (int64_t)blockIdx.x * L;
    for (int e = threadIdx.x; e < L; e += kLayoutThreads) row[e] = hist[e];
}

// Block-wide exclusive scan of one int32 per thread (256 threads).
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t *lds_waves, int32_t *total)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
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
    for (int i = 0; i < kLayoutWaves; ++i) {
        const int32_t s = lds_waves[i];
        if (i < w) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// Kernel 2 (grid = max(1, tiles)): every block derives the per-expert totals
// and its tile's prefix from tile_counts, block 0 publishes counts and
// seg_indptr, and each block ranks its own slots:
//   dst(i) = seg_indptr[e] + sum over earlier tiles of tile_counts[.][e]
//          + slots of e in earlier waves of this tile
//          + slots of e earlier in this wave (ballot / popcount).
// Slot order inside the tile is wave-major, group-major, lane-minor, which is
// the flat slot order, so the ranks are stable.
__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(
    const int32_t *__restrict__ ids, int64_t n, int32_t expert_begin, int32_t L,
    const int32_t *__restrict__ tile_counts, int64_t tiles, int32_t *__restrict__ counts,
    int64_t *__restrict__ seg_indptr, int32_t *__restrict__ src2dst,
    int32_t *__restrict__ reorder)
{
    extern __shared__ int32_t smem[];
    int32_t *base = smem;                 // [L] first row of expert e in this tile
    int32_t *wcnt = smem + L;             // [kLayoutWaves][L]
    __shared__ int32_t scan_tmp[kLayoutWaves];

    const int64_t tile = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;

    // 1. totals and tile prefixes; each thread owns a run of experts
    const int per = (L + kLayoutThreads - 1) / kLayoutThreads;
    const int e0 = tid * per;
    int32_t run_total = 0;
    for (int q = 0; q < per; ++q) {
        const int e = e0 + q;
        if (e >= L) break;
        int32_t tot = 0, pre = 0;
        for (int64_t t = 0; t < tiles; ++t) {
            const int32_t c = tile_counts[t * L + e];
            tot += c;
            pre += (t < tile) ? c : 0;
        }
        base[e] = pre;
        wcnt[e] = tot;                     // scratch: totals, overwritten below
        run_total += tot;
    }
    int32_t R = 0;
    int32_t excl = block_exclusive_scan(run_total, scan_tmp, &R);
    for (int q = 0; q < per; ++q) {
        const int e = e0 + q;
        if (e >= L) break;
        const int32_t tot = wcnt[e];
        if (tile == 0) {
            counts[e] = tot;
            seg_indptr[e] = excl;
        }
        base[e] += excl;
        excl += tot;
    }
    if (tile == 0 && tid == 0) seg_indptr[L] = R;
    __syncthreads();
    for (int idx = tid; idx < kLayoutWaves * L; idx += kLayoutThreads) wcnt[idx] = 0;
    __syncthreads();

    // 2. ranks inside each wave's 256 consecutive slots, 64 at a time
    int32_t *my_cnt = wcnt + w * L;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    int32_t ge[kGroupsPerWave], gr[kGroupsPerWave];
    const int64_t wave_base = tile * kTile + (int64_t)w * kSlotsPerWave;
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {
        const int64_t i = wave_base + g * kWave + lane;
        const int32_t e = (i < n) ? local_expert(ids[i], expert_begin, L) : -1;
        uint64_t pending = __ballot(e >= 0);
        int32_t r = 0;
        while (pending) {
            const int leader = __builtin_ctzll(pending);
            const int32_t el = __builtin_amdgcn_readlane(e, leader);
            const uint64_t m = __ballot(e == el);
            const int32_t before = my_cnt[el];
            if (e == el) r = before + __popcll(m & lt_mask);
            if (lane == leader) my_cnt[el] = before + __popcll(m);
            pending &= ~m;
        }
        ge[g] = e;
        gr[g] = r;
    }
    __syncthreads();

    // 3. wave counts -> wave offsets (in place), seeded with the tile base
    for (int e = tid; e < L; e += kLayoutThreads) {
        int32_t run = base[e];
#pragma unroll
        for (int v = 0; v < kLayoutWaves; ++v) {
            const int32_t c = wcnt[v * L + e];
            wcnt[v * L + e] = run;
            run += c;
        }
    }
    __syncthreads();

    // 4. publish
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {
        const int64_t i = wave_base + g * kWave + lane;
        if (i >= n) continue;
        const int32_t e = ge[g];
        if (e < 0) {
            src2dst[i] = -1;
        } else {
            const int32_t dst = my_cnt[e] + gr[g];
            src2dst[i] = dst;
            reorder[dst] = e;
        }
    }
}

// ---------------------------------------------------------------------------
// normal dispatch: row scatter
// ---------------------------------------------------------------------------

constexpr int kRowThreads = 128;
constexpr int kRowUnroll = 8;        // 16-byte chunks per lane per pass

// One block per token.  Each lane loads up to kRowUnroll 16-byte chunks of
// the row once, then stores them to every valid destination.
__global__ __launch_bounds__(kRowThreads) void scatter_rows_v16(
    const uint4 *__restrict__ x, int64_t chunks, int32_t k,
    const int32_t *__restrict__ src2dst, uint4 *__restrict__ out, int64_t cap_rows,
    int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int32_t *d = src2dst + t * k;
    bool any = false;
    for (int j = 0; j < k; ++j) any |= d[j] >= 0;
    if (!any) return;
    const uint4 *src = x + t * chunks;
    for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)kRowThreads * kRowUnroll) {
        uint4 v[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int64_t c = c0 + u * kRowThreads + threadIdx.x;
            v[u] = (c < chunks) ? src[c] : make_uint4(0, 0, 0, 0);
        }
        for (int j = 0; j < k; ++j) {
            const int32_t dst = d[j];
            if (dst < 0) continue;
            if (dst >= cap_rows) {
                if (c0 == 0 && threadIdx.x == 0) set_status(status, CDL_STATUS_ROWS_OVERFLOW);
                continue;
            }
            uint4 *o = out + (int64_t)dst * chunks;
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int64_t c = c0 + u * kRowThreads + threadIdx.x;
                if (c < chunks) o[c] = v[u];
            }
        }
    }
}

// Any H, any 2-byte alignment: element-wise copy.
__global__ __launch_bounds__(kRowThreads) void scatter_rows_u16(
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
        for (int64_t h = threadIdx.x; h < H; h += kRowThreads) out[(int64_t)dst * H + h] = x[t * H + h];
    }
}

// ---------------------------------------------------------------------------
// fp8 dispatch: per-token group quantisation on the scatter
// ---------------------------------------------------------------------------

// Two fp32 values (already clamped to [-448, 448]) to OCP E4M3FN bytes, round
// to nearest even: v_cvt_pk_fp8_f32, which on gfx950 produces the OCP format.
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float quant_in(float v, float a, float s)
{
    if (a > 0.0f) {
        v = v / s;                      // correctly rounded binary32 division
        v = fminf(fmaxf(v, -448.0f), 448.0f);
    }
    return v;
}

// One block per token.  A group of 128 elements is 16 chunks of 8, held by 16
// consecutive lanes; their amax is reduced with xor shuffles inside the 16.
__global__ __launch_bounds__(kRowThreads) void scatter_rows_fp8(
    const uint4 *__restrict__ x, int64_t chunks, int32_t k, const int32_t *__restrict__ src2dst,
    uint2 *__restrict__ out_q, float *__restrict__ out_s, int64_t groups, int64_t cap_rows,
    int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int32_t *d = src2dst + t * k;
    bool any = false;
    for (int j = 0; j < k; ++j) any |= d[j] >= 0;
    if (!any) return;
    const uint4 *src = x + t * chunks;
    for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)kRowThreads * kRowUnroll) {
        uint2 q[kRowUnroll];
        float sc[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int64_t c = c0 + u * kRowThreads + threadIdx.x;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < chunks) v = src[c];
            float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                          bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e]));
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 16));
            const float s = a / 448.0f;
            uint32_t lo = pack2_e4m3(quant_in(f[0], a, s), quant_in(f[1], a, s)) |
                          (pack2_e4m3(quant_in(f[2], a, s), quant_in(f[3], a, s)) << 16);
            uint32_t hi = pack2_e4m3(quant_in(f[4], a, s), quant_in(f[5], a, s)) |
                          (pack2_e4m3(quant_in(f[6], a, s), quant_in(f[7], a, s)) << 16);
            q[u] = make_uint2(lo, hi);
            sc[u] = s;
        }
        for (int j = 0; j < k; ++j) {
            const int32_t dst = d[j];
            if (dst < 0) continue;
            if (dst >= cap_rows) {
                if (c0 == 0 && threadIdx.x == 0) set_status(status, CDL_STATUS_ROWS_OVERFLOW);
                continue;
            }
            uint2 *oq = out_q + (int64_t)dst * chunks;
            float *os = out_s + (int64_t)dst * groups;
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int64_t c = c0 + u * kRowThreads + threadIdx.x;
                if (c < chunks) {
                    oq[c] = q[u];
                    if ((c & 15) == 0) os[c >> 4] = sc[u];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// low-latency dispatch
// ---------------------------------------------------------------------------

// One block per token: the destination of valid slot i in the padded buffer is
// row e*cap + (src2dst[i] - seg_indptr[e]).  Blocks whose index is below
// ceil(L / threads) also write masked_m; blocks at or beyond T stop there.
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

__global__ __launch_bounds__(kRowThreads) void scatter_rows_ll(
    const uint4 *__restrict__ x, int64_t T, int64_t chunks, int32_t k,
    const int32_t *__restrict__ ids, int32_t expert_begin, int32_t L,
    const int32_t *__restrict__ src2dst, const int64_t *__restrict__ seg_indptr,
    const int32_t *__restrict__ counts, int64_t cap, uint4 *__restrict__ out,
    int32_t *__restrict__ masked_m, int32_t *__restrict__ ll_src2dst,
    int32_t *__restrict__ status)
{
    {
        const int64_t e = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
        if (e < L) masked_m[e] = (int32_t)((int64_t)counts[e] < cap ? counts[e] : cap);
    }
    const int64_t t = blockIdx.x;
    if (t >= T) return;
    bool any = false;
    for (int j = 0; j < k; ++j) {
        const int64_t i = t * k + j;
        bool ovf;
        const int64_t row = ll_row(ids, expert_begin, L, src2dst, seg_indptr, cap, i, &ovf);
        if (threadIdx.x == 0) {
            ll_src2dst[i] = (int32_t)row;
            if (ovf) set_status(status, CDL_STATUS_LL_OVERFLOW);
        }
        any |= row >= 0;
    }
    if (!any) return;
    const uint4 *src = x + t * chunks;
    for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)kRowThreads * kRowUnroll) {
        uint4 v[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int64_t c = c0 + u * kRowThreads + threadIdx.x;
            v[u] = (c < chunks) ? src[c] : make_uint4(0, 0, 0, 0);
        }
        for (int j = 0; j < k; ++j) {
            bool ovf;
            const int64_t row = ll_row(ids, expert_begin, L, src2dst, seg_indptr, cap, t * k + j, &ovf);
            if (row < 0) continue;
            uint4 *o = out + row * chunks;
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int64_t c = c0 + u * kRowThreads + threadIdx.x;
                if (c < chunks) o[c] = v[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// combine: gather + weighted fp32 reduce
// ---------------------------------------------------------------------------

// One block per token.  acc = fma(w_j, y_j, acc) over the valid slots j in
// ascending order from +0 (v_fma_f32 is correctly rounded), one bf16 rounding.
__global__ __launch_bounds__(kRowThreads) void combine_rows_v16(
    const uint4 *__restrict__ y, int64_t y_rows, int64_t chunks, const int32_t *__restrict__ map,
    const float *__restrict__ wts, int32_t k, uint4 *__restrict__ out,
    int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int32_t *m = map + t * k;
    const float *w = wts + t * k;
    for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)kRowThreads * kRowUnroll) {
        float acc[kRowUnroll][8];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int32_t r = m[j];
            if (r < 0) continue;
            if ((int64_t)r >= y_rows) {
                if (c0 == 0 && threadIdx.x == 0) set_status(status, CDL_STATUS_MAP_RANGE);
                continue;
            }
            const float wj = w[j];
            const uint4 *yr = y + (int64_t)r * chunks;
            uint4 v[kRowUnroll];
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int64_t c = c0 + u * kRowThreads + threadIdx.x;
                v[u] = (c < chunks) ? yr[c] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                acc[u][0] = fmaf(wj, bf16_lo(v[u].x), acc[u][0]);
                acc[u][1] = fmaf(wj, bf16_hi(v[u].x), acc[u][1]);
                acc[u][2] = fmaf(wj, bf16_lo(v[u].y), acc[u][2]);
                acc[u][3] = fmaf(wj, bf16_hi(v[u].y), acc[u][3]);
                acc[u][4] = fmaf(wj, bf16_lo(v[u].z), acc[u][4]);
                acc[u][5] = fmaf(wj, bf16_hi(v[u].z), acc[u][5]);
                acc[u][6] = fmaf(wj, bf16_lo(v[u].w), acc[u][6]);
                acc[u][7] = fmaf(wj, bf16_hi(v[u].w), acc[u][7]);
            }
        }
        uint4 *o = out + t * chunks;
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int64_t c = c0 + u * kRowThreads + threadIdx.x;
            if (c < chunks)
                o[c] = make_uint4(pack_bf16_rne(acc[u][0], acc[u][1]), pack_bf16_rne(acc[u][2], acc[u][3]),
                                  pack_bf16_rne(acc[u][4], acc[u][5]), pack_bf16_rne(acc[u][6], acc[u][7]));
        }
    }
}

// Any H, any 2-byte alignment.
__global__ __launch_bounds__(kRowThreads) void combine_rows_u16(
    const uint16_t *__restrict__ y, int64_t y_rows, int64_t H, const int32_t *__restrict__ map,
    const float *__restrict__ wts, int32_t k, uint16_t *__restrict__ out,
    int32_t *__restrict__ status)
{
    const int64_t t = blockIdx.x;
    const int32_t *m = map + t * k;
    const float *w = wts + t * k;
    for (int64_t h = threadIdx.x; h < H; h += kRowThreads) {
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

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

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

inline size_t layout_ws_bytes(int64_t T, int32_t k, int32_t L)
{
    const int64_t tiles = layout_tiles(T * k);
    const size_t bytes = (size_t)tiles * (size_t)L * sizeof(int32_t);
    return ((bytes + 255) & ~(size_t)255) + 256;
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
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (L < 1 || L > CDL_MAX_LOCAL_EXPERTS) return CDL_ERR_BAD_SIZE;
    if (!counts || !seg_indptr) return CDL_ERR_NULL_POINTER;
    if (T > 0 && (!topk_ids || !src2dst || !reorder_topk_ids)) return CDL_ERR_NULL_POINTER;
    const size_t need = layout_ws_bytes(T, k, L);
    if (!ws) return CDL_ERR_NULL_POINTER;
    if (ws_bytes < need) return CDL_ERR_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    const int64_t n = T * k;
    const int64_t tiles = layout_tiles(n);
    int32_t *tile_counts = (int32_t *)ws;
    if (tiles > 0) {
        layout_count_kernel<<<dim3((unsigned)tiles), dim3(kLayoutThreads), L * sizeof(int32_t), s>>>(
            topk_ids, n, expert_begin, L, tile_counts);
        if ((rc = launch_status()) != CDL_OK) return rc;
    }
    const size_t lds = (size_t)(1 + kLayoutWaves) * L * sizeof(int32_t);
    layout_rank_kernel<<<dim3((unsigned)(tiles > 0 ? tiles : 1)), dim3(kLayoutThreads), lds, s>>>(
        topk_ids, n, expert_begin, L, tile_counts, tiles, counts, seg_indptr, src2dst,
        reorder_topk_ids);
    return launch_status();
}

int cdl_dispatch(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *src2dst,
                 uint16_t *out, int64_t cap_rows, int32_t *status, void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap_rows < 0) return CDL_ERR_BAD_SIZE;
    if (T == 0) return CDL_OK;
    if (!x || !src2dst) return CDL_ERR_NULL_POINTER;
    if (cap_rows > 0 && !out) return CDL_ERR_NULL_POINTER;
    if (cap_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    hipStream_t s = (hipStream_t)stream;
    if (H % 8 == 0 && aligned16(x) && aligned16(out)) {
        scatter_rows_v16<<<dim3((unsigned)T), dim3(kRowThreads), 0, s>>>(
            (const uint4 *)x, H / 8, k, src2dst, (uint4 *)out, cap_rows, status);
    } else {
        scatter_rows_u16<<<dim3((unsigned)T), dim3(kRowThreads), 0, s>>>(x, H, k, src2dst, out,
                                                                            cap_rows, status);
    }
    return launch_status();
}

int cdl_dispatch_fp8(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *src2dst,
                     uint8_t *out_q, float *out_scales, int64_t cap_rows, int32_t *status,
                     void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap_rows < 0) return CDL_ERR_BAD_SIZE;
    if (H % CDL_FP8_GROUP != 0) return CDL_ERR_UNSUPPORTED;
    if (T == 0) return CDL_OK;
    if (!x || !src2dst) return CDL_ERR_NULL_POINTER;
    if (cap_rows > 0 && (!out_q || !out_scales)) return CDL_ERR_NULL_POINTER;
    if (cap_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (!aligned16(x) || (cap_rows > 0 && ((uintptr_t)out_q & 7u) != 0) ||
        (cap_rows > 0 && ((uintptr_t)out_scales & 3u) != 0))
        return CDL_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    scatter_rows_fp8<<<dim3((unsigned)T), dim3(kRowThreads), 0, s>>>(
        (const uint4 *)x, H / 8, k, src2dst, (uint2 *)out_q, out_scales, H / CDL_FP8_GROUP,
        cap_rows, status);
    return launch_status();
}

int cdl_dispatch_ll(const uint16_t *x, int64_t T, int64_t H, int32_t k, const int32_t *topk_ids,
                    int32_t expert_begin, int32_t L, const int32_t *src2dst,
                    const int64_t *seg_indptr, const int32_t *counts, int64_t cap, uint16_t *out,
                    int32_t *masked_m, int32_t *ll_src2dst, int32_t *status, void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || cap < 0 || L < 1 || L > CDL_MAX_LOCAL_EXPERTS) return CDL_ERR_BAD_SIZE;
    if (H % 8 != 0) return CDL_ERR_UNSUPPORTED;
    if ((int64_t)L * cap > INT32_MAX) return CDL_ERR_TOO_LARGE;
    if (!counts || !seg_indptr || !masked_m) return CDL_ERR_NULL_POINTER;
    if (T > 0 && (!x || !topk_ids || !src2dst || !ll_src2dst)) return CDL_ERR_NULL_POINTER;
    if (cap > 0 && !out) return CDL_ERR_NULL_POINTER;
    if ((T > 0 && !aligned16(x)) || (cap > 0 && !aligned16(out))) return CDL_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    // one block per token; at least enough blocks to write masked_m
    const int64_t mm_blocks = (L + kRowThreads - 1) / kRowThreads;
    const int64_t grid = T > mm_blocks ? T : mm_blocks;
    scatter_rows_ll<<<dim3((unsigned)grid), dim3(kRowThreads), 0, s>>>(
        (const uint4 *)x, T, H / 8, k, topk_ids, expert_begin, L, src2dst, seg_indptr, counts,
        cap, (uint4 *)out, masked_m, ll_src2dst, status);
    return launch_status();
}

int cdl_combine(const uint16_t *y, int64_t y_rows, int64_t H, const int32_t *map,
                const float *topk_weights, int64_t T, int32_t k, uint16_t *out, int32_t *status,
                void *stream)
{
    int rc = check_tk(T, k);
    if (rc != CDL_OK) return rc;
    if (H < 1 || y_rows < 0) return CDL_ERR_BAD_SIZE;
    if (T == 0) return CDL_OK;
    if (!map || !topk_weights || !out) return CDL_ERR_NULL_POINTER;
    if (y_rows > 0 && !y) return CDL_ERR_NULL_POINTER;
    if (y_rows > INT32_MAX) return CDL_ERR_TOO_LARGE;
    hipStream_t s = (hipStream_t)stream;
    if (H % 8 == 0 && aligned16(y) && aligned16(out)) {
        combine_rows_v16<<<dim3((unsigned)T), dim3(kRowThreads), 0, s>>>(
            (const uint4 *)y, y_rows, H / 8, map, topk_weights, k, (uint4 *)out, status);
    } else {
        combine_rows_u16<<<dim3((unsigned)T), dim3(kRowThreads), 0, s>>>(
            y, y_rows, H, map, topk_weights, k, out, status);
    }
    return launch_status();
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
    default: return "unknown cdl status code";
    }
}

}  // extern "C"
