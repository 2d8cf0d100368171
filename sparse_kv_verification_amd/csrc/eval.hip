// Evaluator of the Dustin translation's section 3.1 for gfx950:
//   A[b][s][j] = (1/H_q) sum_h softmax_j(scale * q[b][s][h] . K[b][j][h/G])
// (full-cache attention weights of each window step, head mean) and the
// attention recovery rate of an index set, Eq. (1) per step and Eq. (2)
// averaged over the window.
//
// The per-row normalisers come from the dense attention kernel (its lse
// output); the probability kernel then streams K once more and writes A.
// Neither kernel is part of the timed verification step.

#include "common.h"
#include "internal.h"

namespace dustin {

constexpr int ECH = 256;   // positions per work-group

template <bool F32, int D>
__global__ __launch_bounds__(256) void window_probs_kernel(WindowArgs a) {
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int LPI = D * ESZ / 16;
    constexpr int EPL = 16 / ESZ;
    constexpr int IPP = 256 / LPI;
    __shared__ float qs[64][D];
    __shared__ float ls[64];
    __shared__ float acc[16][ECH];

    const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const KvView &kv = a.kv;
    const int nb = min(max(kv.seq_lens[b], 0), kv.N_max);
    const int j0 = chunk * ECH;
    const int R = a.w * a.G;
    const int grp = tid / LPI, sl = tid - (tid / LPI) * LPI;

    for (int i = tid; i < a.w * ECH; i += 256) acc[i / ECH][i % ECH] = 0.f;
    for (int g = 0; g < kv.Hkv; ++g) {
        __syncthreads();
        for (int e = tid; e < R * D; e += 256) {
            const int r = e / D, d = e - (e / D) * D;
            const int sq = r / a.G, gh = r - (r / a.G) * a.G;
            const size_t qi = (((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh) * D + d;
            qs[r][d] = F32 ? ((const float *)a.q)[qi] : bf16_bits_to_f32(((const uint16_t *)a.q)[qi]);
        }
        if (tid < R) {
            const int sq = tid / a.G, gh = tid - (tid / a.G) * a.G;
            ls[tid] = a.lse[((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh] * kLog2e;
        }
        __syncthreads();
        for (int pos = grp; pos < ECH; pos += IPP) {
            const int j = j0 + pos;
            if (j >= nb) continue;
            int64_t rr;
            bool ok = true;
            if (kv.page_size == 0) {
                rr = (int64_t)b * kv.N_max + j;
            } else {
                const int pg = kv.page_table[(int64_t)b * kv.max_pages + (j >> 4)];
                ok = pg >= 0 && pg < kv.num_pages;
                rr = ok ? (int64_t)pg * 16 + (j & 15) : 0;
            }
            float x[8];
            if (ok) {
                const u32x4 v = *(const u32x4 *)(kv.k + ((rr * kv.Hkv + g) * D) * ESZ + sl * 16);
                if constexpr (F32) {
                    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
                } else {
                    for (int i = 0; i < 4; ++i) {
                        x[2 * i] = __uint_as_float(v[i] << 16);
                        x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
                    }
                }
            } else {
                for (int i = 0; i < 8; ++i) x[i] = 0.f;
            }
            for (int r = 0; r < R; ++r) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < EPL; ++i) s += qs[r][sl * EPL + i] * x[i];
#pragma unroll
                for (int o = LPI / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
                if (sl == 0 && ok) acc[r / a.G][pos] += exp2f(s * a.scale_log2 - ls[r]);
            }
        }
    }
    __syncthreads();
    const float inv = 1.f / (float)a.Hq;
    for (int i = tid; i < a.w * ECH; i += 256) {
        const int s = i / ECH, pos = i % ECH, j = j0 + pos;
        if (j < kv.N_max) a.A[((size_t)b * a.w + s) * kv.N_max + j] = (j < nb) ? acc[s][pos] * inv : 0.f;
    }
}

hipError_t launch_window_probs(const WindowArgs &a, hipStream_t s) {
    const dim3 grid((a.kv.N_max + ECH - 1) / ECH, a.kv.B);
    if (a.kv.f32) {
        switch (a.kv.D) {
            case 32: hipLaunchKernelGGL((window_probs_kernel<true, 32>), grid, dim3(256), 0, s, a); break;
            case 64: hipLaunchKernelGGL((window_probs_kernel<true, 64>), grid, dim3(256), 0, s, a); break;
            case 128: hipLaunchKernelGGL((window_probs_kernel<true, 128>), grid, dim3(256), 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.kv.D) {
            case 32: hipLaunchKernelGGL((window_probs_kernel<false, 32>), grid, dim3(256), 0, s, a); break;
            case 64: hipLaunchKernelGGL((window_probs_kernel<false, 64>), grid, dim3(256), 0, s, a); break;
            case 128: hipLaunchKernelGGL((window_probs_kernel<false, 128>), grid, dim3(256), 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

// ARR (Eq. 1) per window step and its window mean (Eq. 2).  One work-group
// per sequence; fixed-order tree reduction.
__global__ __launch_bounds__(256) void arr_kernel(ArrArgs a) {
    __shared__ float red[256];
    __shared__ float steps[64];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int nb = min(max(a.seq_lens[b], 0), a.N_max);
    const int cnt = min(max(a.count[b], 0), a.k);
    for (int s = 0; s < a.w; ++s) {
        const float *Ab = a.A + ((size_t)b * a.w + s) * a.N_max;
        float part = 0.f;
        for (int i = tid; i < cnt; i += 256) {
            const int j = a.idx[(size_t)b * a.k + i];
            if (j >= 0 && j < nb) part += Ab[j];
        }
        red[tid] = part;
        __syncthreads();
        for (int o = 128; o >= 1; o >>= 1) {
            if (tid < o) red[tid] += red[tid + o];
            __syncthreads();
        }
        if (tid == 0) {
            steps[s] = red[0];
            if (a.arr_step) a.arr_step[(size_t)b * a.w + s] = red[0];
        }
        __syncthreads();
    }
    if (tid == 0 && a.arr_window) {
        float t = 0.f;
        for (int s = 0; s < a.w; ++s) t += steps[s];
        a.arr_window[b] = t / (float)a.w;
    }
}

hipError_t launch_arr(const ArrArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(arr_kernel, dim3(a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Eq. (3)'s averaged future attention: Abar[b][j] = (1/w) sum_s A[b][s][j],
// summed in window order.
__global__ __launch_bounds__(256) void window_mean_kernel(const float *A, int B, int w, int N, float *Abar) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)B * N) return;
    const int64_t b = e / N, j = e - (e / N) * N;
    const float *a = A + b * w * N + j;
    float t = 0.f;
    for (int s = 0; s < w; ++s) t += a[(int64_t)s * N];
    Abar[e] = t / (float)w;
}

hipError_t launch_window_mean(const float *A, int B, int w, int N, float *Abar, hipStream_t s) {
    const int64_t n = (int64_t)B * N;
    hipLaunchKernelGGL(window_mean_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, A, B, w, N, Abar);
    return hipGetLastError();
}

}  // namespace dustin
