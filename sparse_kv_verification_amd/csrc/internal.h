// Internal interfaces between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace dustin {

// ---------------------------------------------------------------- draft window in the cache
hipError_t launch_append_window(const KvView &kv, const void *k_win, const void *v_win, int w, hipStream_t s);
hipError_t launch_commit_window(int32_t *seq_lens, const int32_t *accepted, int B, int w, hipStream_t s);

// ---------------------------------------------------------------- scoring
constexpr int kScoreChunk = 256;    // positions per scoring work-group
constexpr int kMaxScoreRows = 64;   // scored target rows
constexpr int kMaxDraftLayers = 32;
constexpr int kMaxDraftBatch = 1024;  // sequences per call on the draft side
constexpr int kMaxScoreQoff = 256;   // rows of the float32 draft path

struct ScorePlan {
    int nchunk;                     // ceil(N_max / kScoreChunk)
    // target side
    size_t off_tlogit, off_tstat, off_tlse;   // [B][S][N_max], [B][S][nchunk][2], [B][S]
    // draft side
    size_t off_dstat, off_dlse;     // [B][L_d][Hkv_d][rows][nchunk][2], [B][L_d][Hkv_d][rows]
    int acc_groups;                 // layer groups of the streaming accumulation pass
    size_t off_dpart;               // [acc_groups][B][N_max] partial S_Draft (acc_groups > 1)
    size_t ws_bytes;
};

ScorePlan score_plan(int B, int N_max, int L_d, int H_d, int gamma, int S, int Hkv_d);

struct TargetScoreArgs {
    KvView kv[8];                   // distinct target layers referenced (<= 8)
    int32_t n_layers;
    const void *q_hist;             // [B][S][D]
    int32_t S;
    int32_t row_layer[kMaxScoreRows];   // index into kv[]
    int32_t row_kvh[kMaxScoreRows];     // KV head of each row
    float scale_log2;
    float *s_target;                // [B][N_max]
    float *rows_out;                // [S][B][N_max] per-row probabilities instead of the sum, or NULL
    float *logit;                   // ws
    float *stat;                    // ws
    float *lse;                     // ws
    int32_t nchunk;
};

hipError_t launch_target_score(const TargetScoreArgs &a, hipStream_t s);

struct DraftScoreArgs {
    KvView kv[kMaxDraftLayers];
    int32_t L_d, H_d, gamma, Hkv_d, G_d, rows;  // rows = gamma * G_d
    const void *q_draft;            // [B][L_d][gamma][H_d][d_d]
    float scale_log2;
    float *s_draft;                 // [B][N_max]
    float *stat;                    // ws
    float *lse;                     // ws
    int32_t nchunk;
    float *steps_out;               // window form: [B][gamma][N_max] per-step sums times steps_scale
    float steps_scale;
    // window form on a slice of the window steps, or on steps stored step-
    // major: elements of q_draft per sequence (0: L_d * gamma * H_d * d_d)
    // and between consecutive steps (0: H_d * d_d); rows of steps_out per
    // sequence (0: gamma) and between consecutive steps (0: 1)
    int64_t q_bstride, q_sstride;
    int32_t steps_bstride, steps_sstride;
    float *part;                    // ws: [acc_groups][B][N_max] per-layer-group partial sums
    int32_t acc_groups;             // layer groups of the streaming accumulation (1: no partials)
    // supplied row normalisers, natural log, [B][L_d][gamma][H_d] (nullable):
    // taken instead of the statistics pass
    const float *lse_in;
    // row-normaliser query (nullable): the normalisers are written here in the
    // layout of lse_in and nothing is accumulated
    float *lse_out;
};

hipError_t launch_draft_score(const DraftScoreArgs &a, hipStream_t s);
// Window attention A (Eq. 1) of one layer through the draft passes: bf16,
// gamma <= 4 window steps, gamma * G <= 64 rows; steps_out / steps_scale set
// (and q_bstride / steps_bstride for a slice of a longer window).
hipError_t launch_window_steps(const DraftScoreArgs &a, hipStream_t s);

// ---------------------------------------------------------------- select
struct TopkPlan {
    size_t off_flag;                // [B][N_max] uint8 tier flags
    size_t ws_bytes;
};
TopkPlan topk_plan(int B, int N_max, int k);

struct TopkArgs {
    const float *s_draft, *s_target;
    const int32_t *seq_lens;
    int32_t B, N_max, k, m, n_sink, n_window;
    // row r of a launch reads score row r % d_mod / r % t_mod and length
    // r % len_mod (0: row r itself), so candidates can share a base vector
    int32_t d_mod, t_mod, len_mod;
    int32_t *idx, *count;
    int8_t *tier;
    uint8_t *flag;
};
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);

// ---------------------------------------------------------------- configuration search
hipError_t launch_build_rows(const float *base, const float *units, const int32_t *ids, int C, int B, int N_max,
                             float *out, hipStream_t s);
hipError_t launch_gather_sum(const float *abar, const int32_t *idx, const int32_t *count, int rows, int B, int N_max,
                             int k, float *arr, hipStream_t s);
hipError_t launch_batch_mean(const float *arr, int C, int B, float *mean, hipStream_t s);
hipError_t launch_accumulate(float *dst, const float *src, int64_t n, bool overwrite, hipStream_t s);

// measurement kernels (probe.hip)
hipError_t launch_probe_stream_read(const void *p, size_t bytes, bool nontemporal, uint32_t *sink, int blocks,
                                    hipStream_t s);
hipError_t launch_probe_gather_rows(const void *base, const void *base2, int64_t row_stride, int64_t buf_rows,
                                    const int32_t *rows, int64_t n_rows, int32_t row_bytes, int blocks, hipStream_t s);

// ---------------------------------------------------------------- evaluator
struct WindowArgs {
    KvView kv;
    const void *q;                  // [B][w][Hq][D]
    int32_t w, Hq, G;
    float scale_log2;
    const float *lse;               // [B][w][Hq] natural-log row normalisers
    float *A;                       // [B][w][N_max]
};
hipError_t launch_window_probs(const WindowArgs &a, hipStream_t s);

struct ArrArgs {
    const float *A;
    const int32_t *seq_lens;
    int32_t B, w, N_max, k;
    const int32_t *idx, *count;
    float *arr_step, *arr_window;
};
hipError_t launch_arr(const ArrArgs &a, hipStream_t s);
hipError_t launch_window_mean(const float *A, int B, int w, int N, float *Abar, hipStream_t s);

// ---------------------------------------------------------------- page-level estimator
struct PageArgs {
    KvView kv;
    const void *q;            // [B][w][Hq][D]
    int32_t w, Hq;
    void *kmin, *kmax;        // [B][npages][Hkv][D], kv dtype
    int32_t npages;           // ceil(N_max / 16)
    float scale;
    float *scores;            // [B][npages]
    float *pm;                // [B][2][Hkv * D] scratch: sums of max(q, 0), min(q, 0)
};
hipError_t launch_page_bounds(const PageArgs &a, hipStream_t s);
hipError_t launch_page_scores(const PageArgs &a, hipStream_t s);
constexpr int kPageMaxRow = 4096;   // H_kv * head_dim limit of the page estimator


}  // namespace dustin
