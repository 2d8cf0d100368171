// Interfaces of the verification attention kernel (and the cache view every
// kernel shares), separate from the other kernels' interfaces so that the
// attention kernel's sources are exactly attn.hip, common.h and this file.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dustin {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

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
    // causal form only, or nullptr: the window rows come from these
    // [B][w][Hkv][D] inputs, and split 0 of each (b, g) also writes them into
    // the cache (the append and the attention in one launch)
    const char *k_win, *v_win;
    int32_t trace_slot;      // phase-trace builds only: which trace row this launch fills
};

hipError_t launch_attn(const AttnArgs &a, const AttnPlan &p, hipStream_t s);

}  // namespace dustin
