// Kernels of the offline configuration search (blog section 2.4: a per
// (layer, head) score matrix with its head TopK, greedy target and draft
// selection, and the draft-budget split m, all judged by the windowed ARR of
// translation section 3.1, Eq. 2), for gfx950.
//
// A candidate configuration c yields one verification set per sequence b
// (the select kernels run over C * B rows, row r = c * B + b); its objective
// is the windowed ARR of that set.  Eq. 2 is linear in A, so for the set I
//   (1/w) sum_s sum_{j in I} A[s][j] = sum_{j in I} Abar[j]
// with Abar the window-step mean (averaged over target layers as well when
// the set has to serve several layers): a gather-sum per row.

#include "common.h"
#include "internal.h"

namespace dustin {

// out[r][j] = (base ? base[r % B][j] : 0) + (units ? units[ids[r / B]][r % B][j] : 0);
// one work-group row per candidate row r (grid x), positions strided over grid y.
__global__ __launch_bounds__(256) void build_rows_kernel(const float *base, const float *units, const int32_t *ids,
                                                        int B, int N_max, float *out) {
    const int r = blockIdx.x, b = r % B, c = r / B;
    const float *bp = base ? base + (int64_t)b * N_max : nullptr;
    const float *up = units ? units + ((int64_t)ids[c] * B + b) * N_max : nullptr;
    float *op = out + (int64_t)r * N_max;
    for (int j = blockIdx.y * 256 + threadIdx.x; j < N_max; j += gridDim.y * 256) {
        float v = 0.f;
        if (bp) v += bp[j];
        if (up) v += up[j];
        op[j] = v;
    }
}

// arr[r] = sum_{t < count[r]} abar[r % B][idx[r][t]]  (one wave per row, lane
// partials in a fixed order, then the wave sum: deterministic).
__global__ __launch_bounds__(256) void gather_sum_kernel(const float *abar, const int32_t *idx, const int32_t *count,
                                                        int rows, int B, int N_max, int k, float *arr) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (r >= rows) return;
    const float *ab = abar + (int64_t)(r % B) * N_max;
    const int32_t *ix = idx + (int64_t)r * k;
    const int cnt = min(max(count[r], 0), k);
    float acc = 0.f;
    for (int t = lane; t < cnt; t += 64) {
        const int j = ix[t];
        if (j >= 0 && j < N_max) acc += ab[j];
    }
    acc = wave_sum(acc);
    if (lane == 0) arr[r] = acc;
}

// mean[c] = (1/B) sum_b arr[c][b], summed in b order.
__global__ __launch_bounds__(256) void batch_mean_kernel(const float *arr, int C, int B, float *mean) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += arr[(int64_t)c * B + b];
    mean[c] = s / (float)B;
}

// dst[i] = (overwrite ? 0 : dst[i]) + src[i]
__global__ __launch_bounds__(256) void accumulate_kernel(float *dst, const float *src, int64_t n, int overwrite) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = (overwrite ? 0.f : dst[i]) + (src ? src[i] : 0.f);
}

hipError_t launch_build_rows(const float *base, const float *units, const int32_t *ids, int C, int B, int N_max,
                             float *out, hipStream_t s) {
    const dim3 grid((unsigned)(C * B), (unsigned)std::min((N_max + 255) / 256, 64));
    hipLaunchKernelGGL(build_rows_kernel, grid, dim3(256), 0, s, base, units, ids, B, N_max, out);
    return hipGetLastError();
}

hipError_t launch_gather_sum(const float *abar, const int32_t *idx, const int32_t *count, int rows, int B, int N_max,
                             int k, float *arr, hipStream_t s) {
    hipLaunchKernelGGL(gather_sum_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, abar, idx, count, rows, B, N_max, k,
                       arr);
    return hipGetLastError();
}

hipError_t launch_batch_mean(const float *arr, int C, int B, float *mean, hipStream_t s) {
    hipLaunchKernelGGL(batch_mean_kernel, dim3((C + 255) / 256), dim3(256), 0, s, arr, C, B, mean);
    return hipGetLastError();
}

hipError_t launch_accumulate(float *dst, const float *src, int64_t n, bool overwrite, hipStream_t s) {
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(accumulate_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, dst, src, n,
                       overwrite ? 1 : 0);
    return hipGetLastError();
}

}  // namespace dustin
