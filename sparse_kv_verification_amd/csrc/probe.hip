// Measurement kernels: the achievable HBM rates that the step's kernels are
// compared with, beside the 8 TB/s peak.  They compute nothing of the method.
//
//   probe_stream_read   every 16-byte piece of a buffer read once (grid-
//                       stride, four loads in flight per lane), with the
//                       nontemporal policy the scoring passes use or the
//                       default one;
//   probe_gather_rows   rows of `row_bytes` bytes at listed row numbers
//                       gathered into an LDS ring with global->LDS DMA, the
//                       way the verification attention fetches the selected
//                       K and V rows (one 8-wave work-group per CU, a four-
//                       stage ring of 32 KiB, no arithmetic on the data).
//
// The read probe keeps its loads alive by folding the data into a value
// that is written to `sink` only if it equals an impossible marker; the
// DMA of the gather probe writes LDS and cannot be dropped.

#include "common.h"
#include "internal.h"

namespace dustin {

constexpr uint32_t kProbeMarker = 0x9e3779b9u;

template <bool NT>
__global__ __launch_bounds__(256) void probe_stream_read(const u32x4 *p, size_t n, uint32_t *sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * 1024;
    for (size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x; i < n; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t j = i + (size_t)u * 256;
            v[u] = j < n ? (NT ? __builtin_nontemporal_load(p + j) : p[j]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == kProbeMarker) sink[blockIdx.x] = acc;
}

// Wait until this wave's DMA of the current stage has landed while the
// `ahead` stages issued after it (4 instructions each) stay in flight.
template <int A>
__device__ __forceinline__ void probe_wait(int ahead) {
    if constexpr (A <= 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= A) wait_vmcnt<A * 4>();
        else probe_wait<A - 1>(ahead);
    }
}

constexpr int kProbeMaxRowsPerGroup = 4096;

// Work-group g gathers rows [g * per, (g + 1) * per) of `rows` (row numbers
// clamped to [0, buf_rows)), of base and, when given, of base2 at the same
// row numbers.  The group's row numbers are staged in LDS first, so the DMA
// loop issues no other vector-memory load.
__global__ __launch_bounds__(512, 1) void probe_gather_rows(const char *base, const char *base2, int64_t row_stride,
                                                           int64_t buf_rows, const int32_t *rows, int64_t n_rows,
                                                           int32_t row_bytes, int64_t per) {
    constexpr int NBUF = 4;
    constexpr int STAGE = 32 * 1024;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF][STAGE];
    __shared__ int rowtab[kProbeMaxRowsPerGroup];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int cpr = row_bytes / 16;                   // 16-byte pieces per row
    const int ntens = base2 ? 2 : 1;
    const int rows_per_stage = STAGE / (row_bytes * ntens);
    const int64_t r0 = (int64_t)blockIdx.x * per;
    const int64_t r1 = r0 + per < n_rows ? r0 + per : n_rows;
    const int nr = r1 > r0 ? (int)(r1 - r0) : 0;
    for (int t = tid; t < nr; t += 512) {
        const int64_t v = rows[r0 + t];
        rowtab[t] = (int)(v < 0 ? 0 : (v >= buf_rows ? buf_rows - 1 : v));
    }
    wait_vmcnt<0>();
    lds_barrier();
    const int nst = (nr + rows_per_stage - 1) / rows_per_stage;
    // DMA instruction c of a stage (64 lanes x 16 bytes) covers pieces
    // c * 64 .. + 63: piece q is slice q mod cpr of row (q / cpr) mod
    // rows_per_stage of tensor q / (rows_per_stage * cpr).  Each wave issues
    // the 4 instructions c = wave, wave + 8, wave + 16, wave + 24.
    auto issue = [&](int st, int buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = wave + 8 * u;
            const int q = c * 64 + lane;
            const int t = q / (rows_per_stage * cpr);
            const int rl = st * rows_per_stage + (q / cpr) % rows_per_stage;
            const int row = rowtab[rl < nr ? rl : 0];
            const char *src = (t ? base2 : base) + (int64_t)row * row_stride + (q % cpr) * 16;
            dma16_stream(src, &ring[buf][c * 1024]);
        }
    };
    for (int st = 0; st < NBUF - 1 && st < nst; ++st) issue(st, st);
    for (int st = 0; st < nst; ++st) {
        probe_wait<NBUF - 2>(min(nst - 1 - st, NBUF - 2));
        lds_barrier();   // every wave is past stage st - 1: its buffer is free
        if (st + NBUF - 1 < nst) issue(st + NBUF - 1, (st + NBUF - 1) % NBUF);
    }
    wait_vmcnt<0>();
}

hipError_t launch_probe_stream_read(const void *p, size_t bytes, bool nontemporal, uint32_t *sink, int blocks,
                                    hipStream_t s) {
    const size_t n = bytes / 16;
    if (nontemporal)
        hipLaunchKernelGGL(probe_stream_read<true>, dim3(blocks), dim3(256), 0, s, (const u32x4 *)p, n, sink);
    else
        hipLaunchKernelGGL(probe_stream_read<false>, dim3(blocks), dim3(256), 0, s, (const u32x4 *)p, n, sink);
    return hipGetLastError();
}

hipError_t launch_probe_gather_rows(const void *base, const void *base2, int64_t row_stride, int64_t buf_rows,
                                    const int32_t *rows, int64_t n_rows, int32_t row_bytes, int blocks, hipStream_t s) {
    const int64_t per = (n_rows + blocks - 1) / blocks;
    if (per > kProbeMaxRowsPerGroup) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_gather_rows, dim3(blocks), dim3(512), 0, s, (const char *)base, (const char *)base2,
                       row_stride, buf_rows, rows, n_rows, row_bytes, per);
    return hipGetLastError();
}

}  // namespace dustin
