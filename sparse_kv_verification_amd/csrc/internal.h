// Internal interfaces between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dustin {

// Device-side view of one layer's KV cache (see dustin_kv in dustin.h).
struct KvView {
    const char *k;
    const char *v;
    const int32_t *seq_lens;
    const int32_t *page_table;
    int32_t B, Hkv, D, N_max;
    int32_t page_size, max_pages, num_pages;
    int32_t f32;  // 1 = float32 storage, 0 = bfloat16
};

// ---------------------------------------------------------------- attention
constexpr int kAttnTile = 32;            // tokens per tile (float32 kernel; bf16 minimum)
constexpr int kAttnSplitQuantum = 128;   // bf16 splits hold a multiple of this many tokens
constexpr int kAttnMaxTps = 4096;        // tokens per split (row table in LDS)
constexpr int kAttnRingBytes = 128 * 1024;   // LDS of the bf16 kernel's K/V ring
constexpr int kAttnTargetGroups = 256;   // bf16 work-groups the split planner aims for
// Arrival counters occupy a fixed region at the start of every attention
// workspace, one slot per (sequence, KV head), whatever the call's shape: a
// workspace reused by calls of different shapes then never finds a counter
// on top of another call's stored partials.
constexpr int kAttnCounterSlots = 16384;

struct AttnPlan {
    int rows;      // R = w * G query rows per (sequence, KV head)
    int rb;        // 16-row blocks
    int rpad;      // 16 * rb
    int splits;    // token splits per (sequence, KV head)
    int tps;       // tokens per split (multiple of kAttnTile)
    size_t off_m, off_l, off_o;  // workspace byte offsets
    size_t ws_bytes;
};

AttnPlan attn_plan(int B, int w, int Hq, int Hkv, int D, int tokens, bool f32);

struct AttnArgs {
    KvView kv;
    const void *q;           // [B][w][Hq][D]
    int32_t w, Hq, G, R;
    const int32_t *idx;      // [B][k] or nullptr (dense)
    const int32_t *count;    // [B]
    int32_t k;
    float scale_log2;        // softmax scale * log2(e)
    void *out;               // [B][w][Hq][D]
    float *lse;              // [B][w][Hq] or nullptr
    float *part_m, *part_l, *part_o;
    int32_t *counters;       // [B * Hkv]
    int32_t splits, tps, rpad;
    int32_t causal;          // 1: the w window rows after the history are attended causally
};

hipError_t launch_attn(const AttnArgs &a, const AttnPlan &p, hipStream_t s);

// ---------------------------------------------------------------- draft window in the cache
hipError_t launch_append_window(const KvView &kv, const void *k_win, const void *v_win, int w, hipStream_t s);
hipError_t launch_commit_window(int32_t *seq_lens, const int32_t *accepted, int B, int w, hipStream_t s);

// ---------------------------------------------------------------- scoring
constexpr int kScoreChunk = 256;    // positions per scoring work-group
constexpr int kMaxScoreRows = 64;   // scored target rows
constexpr int kMaxDraftLayers = 32;
constexpr int kMaxScoreQoff = 256;   // rows of the float32 draft path

struct ScorePlan {
    int nchunk;                     // ceil(N_max / kScoreChunk)
    // target side
    size_t off_tlogit, off_tstat, off_tlse;   // [B][S][N_max], [B][S][nchunk][2], [B][S]
    // draft side
    size_t off_dstat, off_dlse;     // [B][L_d][Hkv_d][rows][nchunk][2], [B][L_d][Hkv_d][rows]
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
};

hipError_t launch_draft_score(const DraftScoreArgs &a, hipStream_t s);

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

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dustin
