// The draft window in the target cache (Dustin blog, Fig. 5, Stage 2): the
// w draft tokens' keys and values are written right after each sequence's
// history before they are verified, and after verification the accepted
// ones stay: the history length grows by the accepted count, the rows of
// rejected tokens lie past the new length and are overwritten next step.

#include "common.h"
#include "internal.h"

namespace dustin {

// One work-group per (window token t, sequence b); threads copy 16-byte
// pieces of the token's H_kv * head_dim keys and values.
__global__ __launch_bounds__(256) void append_window_kernel(KvView kv, const char *k_win, const char *v_win, int w) {
    const int t = blockIdx.x, b = blockIdx.y;
    const int nb = min(max(kv.seq_lens[b], 0), kv.N_max);
    const int pos = nb + t;
    if (pos >= kv.N_max) return;
    int64_t row;
    if (kv.page_size == 0) {
        row = (int64_t)b * kv.N_max + pos;
    } else {
        const int pg = kv.page_table[(int64_t)b * kv.max_pages + (pos >> 4)];
        if (pg < 0 || pg >= kv.num_pages) return;
        row = (int64_t)pg * 16 + (pos & 15);
    }
    const int esz = kv.f32 ? 4 : 2;
    const int nbytes = kv.Hkv * kv.D * esz;   // a multiple of 16 (head_dim >= 8 for bf16, >= 4 for f32)
    const int64_t src = ((int64_t)b * w + t) * nbytes;
    char *kd = const_cast<char *>(kv.k) + row * nbytes;
    char *vd = const_cast<char *>(kv.v) + row * nbytes;
    for (int o = threadIdx.x * 16; o < nbytes; o += blockDim.x * 16) {
        *(u32x4 *)(kd + o) = *(const u32x4 *)(k_win + src + o);
        *(u32x4 *)(vd + o) = *(const u32x4 *)(v_win + src + o);
    }
}

__global__ void commit_window_kernel(int32_t *seq_lens, const int32_t *accepted, int B, int w) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) seq_lens[b] += min(max(accepted[b], 0), w);
}

hipError_t launch_append_window(const KvView &kv, const void *k_win, const void *v_win, int w, hipStream_t s) {
    hipLaunchKernelGGL(append_window_kernel, dim3(w, kv.B), dim3(256), 0, s, kv, (const char *)k_win,
                       (const char *)v_win, w);
    return hipGetLastError();
}

hipError_t launch_commit_window(int32_t *seq_lens, const int32_t *accepted, int B, int w, hipStream_t s) {
    hipLaunchKernelGGL(commit_window_kernel, dim3((B + 255) / 256), dim3(256), 0, s, seq_lens, accepted, B, w);
    return hipGetLastError();
}

}  // namespace dustin
