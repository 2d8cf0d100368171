// The page-level estimator the pages compare Dustin's scoring with (Quest,
// in the translation's related work: the full cache stays, and KV pages are
// scored from cheap min/max key statistics instead of exact QK^T; Quest-16
// in the blog's Fig. 8), for gfx950:
//
//   kmin[b][p][g][d] = min over positions j of page p (j < n_b) of K[b][j][g][d]
//   kmax[b][p][g][d] = max over the same positions
//   score[b][p] = scale * sum_{s, h} sum_d max(q[b][s][h][d] kmin[b][p][g(h)][d],
//                                              q[b][s][h][d] kmax[b][p][g(h)][d])
//   (0 for pages with no position below n_b)
//
// (the per-head box bound of scale * q . k over the page, summed over the
// window steps and query heads for one global page set).  Pages hold 16
// positions, the cache's own pages when it is paged.

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace dustin {

// One work-group per (page, sequence); each thread takes 16-byte pieces of
// the H_kv * D key values of a position and keeps their running min / max
// over the page's valid positions.  min/max of stored values is exact, so
// the bounds are stored back in the cache dtype without rounding.
template <bool F32>
__global__ __launch_bounds__(256) void page_bounds_kernel(PageArgs a) {
    using T = typename std::conditional<F32, float, uint16_t>::type;
    constexpr int EPV = 16 / sizeof(T);   // elements per 16-byte piece
    const int p = blockIdx.x, b = blockIdx.y;
    const KvView &kv = a.kv;
    const int nb = min(max(kv.seq_lens[b], 0), kv.N_max);
    const int j0 = p * 16;
    const int nrow = max(0, min(16, nb - j0));
    const int row_elems = kv.Hkv * kv.D;
    T *mn = (T *)a.kmin + ((int64_t)b * a.npages + p) * row_elems;
    T *mx = (T *)a.kmax + ((int64_t)b * a.npages + p) * row_elems;
    // physical rows of the page's valid positions (paged: the cache's own page)
    int64_t row0 = -1;
    if (nrow > 0) {
        if (kv.page_size == 0) {
            row0 = (int64_t)b * kv.N_max + j0;
        } else {
            const int pg = kv.page_table[(int64_t)b * kv.max_pages + p];
            row0 = (pg >= 0 && pg < kv.num_pages) ? (int64_t)pg * 16 : -1;
        }
    }
    for (int e = threadIdx.x * EPV; e < row_elems; e += blockDim.x * EPV) {
        float lo[EPV], hi[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            lo[i] = __builtin_huge_valf();
            hi[i] = -__builtin_huge_valf();
        }
        if (row0 >= 0) {
            for (int t = 0; t < nrow; ++t) {
                const u32x4 v = *(const u32x4 *)((const T *)kv.k + (row0 + t) * row_elems + e);
                const T *x = (const T *)&v;
#pragma unroll
                for (int i = 0; i < EPV; ++i) {
                    float f;
                    if constexpr (F32) f = x[i];
                    else f = __builtin_bit_cast(float, (uint32_t)x[i] << 16);
                    lo[i] = fminf(lo[i], f);
                    hi[i] = fmaxf(hi[i], f);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPV; ++i) lo[i] = hi[i] = 0.f;   // no valid position: unused, written as 0
        }
        u32x4 vlo, vhi;
        T *ol = (T *)&vlo, *oh = (T *)&vhi;
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            if constexpr (F32) {
                ol[i] = lo[i];
                oh[i] = hi[i];
            } else {   // exact: the values are bf16 values
                ol[i] = (uint16_t)(__builtin_bit_cast(uint32_t, lo[i]) >> 16);
                oh[i] = (uint16_t)(__builtin_bit_cast(uint32_t, hi[i]) >> 16);
            }
        }
        *(u32x4 *)(mn + e) = vlo;
        *(u32x4 *)(mx + e) = vhi;
    }
}

// Page scores.  Each term splits exactly as
//   max(q lo, q hi) = max(q, 0) hi + min(q, 0) lo                (hi >= lo),
// so, summed over the window steps and the query heads of KV head g,
//   score[p] = scale * sum_{g, d} (P[g][d] hi[p][g][d] + M[g][d] lo[p][g][d])
// with P = sum max(q, 0) and M = sum min(q, 0) over those (step, head)
// pairs: a dot product of the page's bounds with two per-sequence vectors.
// A small kernel forms P and M once per call; the scoring kernel streams the
// bounds once at the HBM rate.

// P / M: work-group (sequence, KV head); thread t takes the 16-byte query
// piece t % (D / EPV) of rows t / (D / EPV), t / (D / EPV) + replicas, ...;
// the replicas are added in LDS.
template <bool F32>
__global__ __launch_bounds__(256) void page_query_split_kernel(PageArgs a) {
    using T = typename std::conditional<F32, float, uint16_t>::type;
    constexpr int EPV = 16 / sizeof(T);
    __shared__ float red[2][256 * EPV];         // [replica][D] partial sums, D / EPV * replicas = 256
    const int b = blockIdx.x, g = blockIdx.y;
    const int D = a.kv.D, G = a.Hq / a.kv.Hkv, nq = a.w * G;
    const int dp = D / EPV, reps = blockDim.x / dp;   // dp divides 256
    const int piece = threadIdx.x % dp, r = threadIdx.x / dp;
    float sp[EPV], sm[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k) sp[k] = sm[k] = 0.f;
    constexpr int U = 4;                        // rows loaded together (one round of independent loads)
    for (int i0 = r; i0 < nq; i0 += U * reps) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = min(i0 + u * reps, nq - 1);
            const int s = i / G, h = g * G + (i - s * G);
            v[u] = *(const u32x4 *)((const T *)a.q + (((int64_t)b * a.w + s) * a.Hq + h) * D + piece * EPV);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u * reps >= nq) break;
            const T *x = (const T *)&v[u];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                float qv;
                if constexpr (F32) qv = x[k];
                else qv = __builtin_bit_cast(float, (uint32_t)x[k] << 16);
                sp[k] += fmaxf(qv, 0.f);
                sm[k] += fminf(qv, 0.f);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
        red[0][r * D + piece * EPV + k] = sp[k];
        red[1][r * D + piece * EPV + k] = sm[k];
    }
    __syncthreads();
    const int rowe = a.kv.Hkv * D;
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
        float p = 0.f, m = 0.f;
        for (int q = 0; q < reps; ++q) {
            p += red[0][q * D + e];
            m += red[1][q * D + e];
        }
        a.pm[((int64_t)b * 2) * rowe + g * D + e] = p;
        a.pm[((int64_t)b * 2 + 1) * rowe + g * D + e] = m;
    }
}

// Scoring: each wave holds P / M for its own row pieces in registers (lane l
// owns the 16-byte pieces l, l + 64, ..., PPL of them) and takes chunks of PC
// pages (PC * PPL = 8: one round of 16 loads per lane per chunk, few enough
// registers for four waves per SIMD to overlap loads with arithmetic); each
// page's sum is reduced across the wave.
#ifndef DUSTIN_PAGE_AUX
#define DUSTIN_PAGE_AUX 2
#endif
constexpr int kPageAux = DUSTIN_PAGE_AUX;   // cache policy of the bounds loads (2: non-temporal, read once)

template <bool F32, int PPL>
__global__ __launch_bounds__(256) void page_scores_kernel(PageArgs a) {
    using T = typename std::conditional<F32, float, uint16_t>::type;
    constexpr int EPV = 16 / sizeof(T);
    constexpr int PC = PPL >= 8 ? 1 : 8 / PPL;  // pages per chunk
    const int b = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const KvView &kv = a.kv;
    const int rowe = kv.Hkv * kv.D, npc = rowe / EPV;
    auto f = [](T x) -> float {
        if constexpr (F32) return x;
        else return __builtin_bit_cast(float, (uint32_t)x << 16);
    };
    // buffer resources over the sequence's bounds (reads past them return 0);
    // the page offset is wave-uniform, lanes add one 32-bit piece offset
    const uint32_t seq_bytes = (uint32_t)((size_t)a.npages * rowe * sizeof(T));
    const __amdgpu_buffer_rsrc_t rmin = __builtin_amdgcn_make_buffer_rsrc(
        (char *)a.kmin + (int64_t)b * seq_bytes, (short)0, (int)seq_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rmax = __builtin_amdgcn_make_buffer_rsrc(
        (char *)a.kmax + (int64_t)b * seq_bytes, (short)0, (int)seq_bytes, 0x00020000);
    uint32_t loff[PPL];
#pragma unroll
    for (int j = 0; j < PPL; ++j) loff[j] = (uint32_t)min(lane + 64 * j, npc - 1) * 16u;
    float pv[PPL][EPV], mv[PPL][EPV];
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
        const int pc = lane + 64 * j;
        const bool ok = pc < npc;
        const float *src = a.pm + (int64_t)b * 2 * rowe + (ok ? pc : 0) * EPV;
#pragma unroll
        for (int k = 0; k < EPV; k += 4) {
            const f32x4 x = *(const f32x4 *)(src + k), y = *(const f32x4 *)(src + rowe + k);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pv[j][k + u] = ok ? x[u] : 0.f;
                mv[j][k + u] = ok ? y[u] : 0.f;
            }
        }
    }
    const int nb = min(max(kv.seq_lens[b], 0), kv.N_max);
    const int used = (nb + 15) / 16;            // pages with positions below n_b
    const int nchunk = (a.npages + PC - 1) / PC;
    float *out = a.scores + (int64_t)b * a.npages;
    for (int c = blockIdx.x * 4 + wave; c < nchunk; c += gridDim.x * 4) {
        const int p0 = c * PC;
        if (p0 >= used) {                       // nothing of the sequence here
            if (lane < PC && p0 + lane < a.npages) out[p0 + lane] = 0.f;
            continue;
        }
        u32x4 vlo[PC][PPL], vhi[PC][PPL];
#pragma unroll
        for (int i = 0; i < PC; ++i) {
            const int pb = min(p0 + i, a.npages - 1) * rowe * (int)sizeof(T);
#pragma unroll
            for (int j = 0; j < PPL; ++j) {
                vlo[i][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rmin, loff[j], pb, kPageAux));
                vhi[i][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rmax, loff[j], pb, kPageAux));
            }
        }
        float acc[PC];
#pragma unroll
        for (int i = 0; i < PC; ++i) {
            acc[i] = 0.f;
#pragma unroll
            for (int j = 0; j < PPL; ++j) {
                const T *lo = (const T *)&vlo[i][j], *hi = (const T *)&vhi[i][j];
#pragma unroll
                for (int k = 0; k < EPV; ++k) acc[i] = fmaf(pv[j][k], f(hi[k]), fmaf(mv[j][k], f(lo[k]), acc[i]));
            }
        }
#pragma unroll
        for (int i = 0; i < PC; ++i) {
            const float v = wave_sum(acc[i]);
            const int p = p0 + i;
            if (lane == 0 && p < a.npages) out[p] = (p < used) ? v * a.scale : 0.f;
        }
    }
}

int page_pieces_per_lane(int Hkv, int D, bool f32) {
    const int npc = Hkv * D / (f32 ? 4 : 8);
    int ppl = 1;
    while (ppl * 64 < npc) ppl *= 2;
    return ppl;
}

hipError_t launch_page_bounds(const PageArgs &a, hipStream_t s) {
    const dim3 grid(a.npages, a.kv.B);
    if (a.kv.f32) hipLaunchKernelGGL(page_bounds_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(page_bounds_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_page_scores(const PageArgs &a, hipStream_t s) {
    if (a.kv.f32) hipLaunchKernelGGL(page_query_split_kernel<true>, dim3(a.kv.B, a.kv.Hkv), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(page_query_split_kernel<false>, dim3(a.kv.B, a.kv.Hkv), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ppl = page_pieces_per_lane(a.kv.Hkv, a.kv.D, a.kv.f32);
    const int pc = ppl >= 8 ? 1 : 8 / ppl;
    const int nchunk = (a.npages + pc - 1) / pc;
    // about 1024 work-groups in all (four waves per SIMD), each wave holding at least one chunk
    const int gx = std::max(1, std::min((1024 + a.kv.B - 1) / a.kv.B, (nchunk + 3) / 4));
    const dim3 grid(gx, a.kv.B);
    // H_kv * head_dim <= 4096: up to 16 pieces per lane in float32, 8 in bfloat16
#define DUSTIN_PAGE_CASE(F, P) \
    case P: hipLaunchKernelGGL((page_scores_kernel<F, P>), grid, dim3(256), 0, s, a); break;
    if (a.kv.f32) {
        switch (ppl) {
            DUSTIN_PAGE_CASE(true, 1) DUSTIN_PAGE_CASE(true, 2) DUSTIN_PAGE_CASE(true, 4)
            DUSTIN_PAGE_CASE(true, 8) DUSTIN_PAGE_CASE(true, 16)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (ppl) {
            DUSTIN_PAGE_CASE(false, 1) DUSTIN_PAGE_CASE(false, 2) DUSTIN_PAGE_CASE(false, 4)
            DUSTIN_PAGE_CASE(false, 8)
            default: return hipErrorInvalidValue;
        }
    }
#undef DUSTIN_PAGE_CASE
    return hipGetLastError();
}

}  // namespace dustin
