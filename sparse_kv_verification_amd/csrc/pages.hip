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
//   max(q lo, q hi) = q (lo + hi) / 2 + |q| (hi - lo) / 2      (hi >= lo),
// so, summed over the window steps and the query heads of KV head g,
//   score[p] = scale * sum_{g, d} (c1[g][d] (lo + hi) + c2[g][d] (hi - lo))
// with c1 = sum q / 2 and c2 = sum |q| / 2 over those (step, head) pairs: a
// dot product of the page's bounds with two per-sequence vectors, so the
// kernel streams the bounds once at the HBM rate.
//
// Work-group (chunk set, sequence): first c1 / c2 into LDS (16-byte query
// pieces, the (step, head) rows split over replicas of the piece grid and
// added up afterwards), then each wave takes chunks of 8 pages; lane l takes
// the row's 16-byte pieces l, l + 64, ... of all 8 pages (16 loads in flight
// per piece), and each page's sum is reduced across the wave.
template <bool F32>
__global__ __launch_bounds__(256) void page_scores_kernel(PageArgs a) {
    using T = typename std::conditional<F32, float, uint16_t>::type;
    constexpr int EPV = 16 / sizeof(T);
    constexpr int PC = 8;                       // pages per chunk
    extern __shared__ float lds[];              // part [R][2][rowe], then c [2][rowe]
    const int b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const KvView &kv = a.kv;
    const int D = kv.D, rowe = kv.Hkv * D, npc = rowe / EPV;
    const int G = a.Hq / kv.Hkv, nq = a.w * G;  // (step, head) rows per KV head
    const int R = max(1, min(nq, (int)blockDim.x / npc));
    float *part = lds, *cc = lds + (size_t)R * 2 * rowe;
    auto f = [](T x) -> float {
        if constexpr (F32) return x;
        else return __builtin_bit_cast(float, (uint32_t)x << 16);
    };
    for (int t = threadIdx.x; t < npc * R; t += blockDim.x) {
        const int pc = t % npc, r = t / npc;
        const int e = pc * EPV, g = e / D, d = e - g * D;   // a piece stays inside one head (D % EPV == 0)
        float s1[EPV], s2[EPV];
#pragma unroll
        for (int k = 0; k < EPV; ++k) s1[k] = s2[k] = 0.f;
        for (int i = r; i < nq; i += R) {
            const int s = i / G, h = g * G + (i - s * G);
            const u32x4 v = *(const u32x4 *)((const T *)a.q + (((int64_t)b * a.w + s) * a.Hq + h) * D + d);
            const T *x = (const T *)&v;
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float qv = f(x[k]);
                s1[k] += qv;
                s2[k] += fabsf(qv);
            }
        }
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
            part[((size_t)r * 2) * rowe + e + k] = s1[k];
            part[((size_t)r * 2 + 1) * rowe + e + k] = s2[k];
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < rowe; e += blockDim.x) {
        float s1 = 0.f, s2 = 0.f;
        for (int r = 0; r < R; ++r) {
            s1 += part[((size_t)r * 2) * rowe + e];
            s2 += part[((size_t)r * 2 + 1) * rowe + e];
        }
        cc[e] = 0.5f * s1;
        cc[rowe + e] = 0.5f * s2;
    }
    __syncthreads();

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
        float acc[PC];
#pragma unroll
        for (int i = 0; i < PC; ++i) acc[i] = 0.f;
        for (int pc = lane; pc < npc; pc += 64) {
            const int e = pc * EPV;
            u32x4 vlo[PC], vhi[PC];
#pragma unroll
            for (int i = 0; i < PC; ++i) {
                const int p = min(p0 + i, a.npages - 1);
                const int64_t off = ((int64_t)b * a.npages + p) * rowe + e;
                vlo[i] = *(const u32x4 *)((const T *)a.kmin + off);
                vhi[i] = *(const u32x4 *)((const T *)a.kmax + off);
            }
            float c1[EPV], c2[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                c1[k] = cc[e + k];
                c2[k] = cc[rowe + e + k];
            }
#pragma unroll
            for (int i = 0; i < PC; ++i) {
                const T *lo = (const T *)&vlo[i], *hi = (const T *)&vhi[i];
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float l = f(lo[k]), h = f(hi[k]);
                    acc[i] = fmaf(c1[k], l + h, acc[i]);
                    acc[i] = fmaf(c2[k], h - l, acc[i]);
                }
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

size_t page_scores_lds_bytes(int Hkv, int D, int w, int Hq, bool f32) {
    const int epv = f32 ? 4 : 8, rowe = Hkv * D, npc = rowe / epv;
    const int R = std::max(1, std::min(w * (Hq / Hkv), 256 / npc));
    return ((size_t)R * 2 + 2) * rowe * sizeof(float);
}

hipError_t launch_page_bounds(const PageArgs &a, hipStream_t s) {
    const dim3 grid(a.npages, a.kv.B);
    if (a.kv.f32) hipLaunchKernelGGL(page_bounds_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(page_bounds_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_page_scores(const PageArgs &a, hipStream_t s) {
    const size_t lds = page_scores_lds_bytes(a.kv.Hkv, a.kv.D, a.w, a.Hq, a.kv.f32);
    const int nchunk = (a.npages + 7) / 8;
    // about 512 work-groups in all, each wave holding at least one chunk
    const int gx = std::max(1, std::min((512 + a.kv.B - 1) / a.kv.B, (nchunk + 3) / 4));
    const dim3 grid(gx, a.kv.B);
    const void *fn = a.kv.f32 ? (const void *)page_scores_kernel<true> : (const void *)page_scores_kernel<false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (a.kv.f32) hipLaunchKernelGGL(page_scores_kernel<true>, grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL(page_scores_kernel<false>, grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace dustin
