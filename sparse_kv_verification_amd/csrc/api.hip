// C ABI of the sparse-verification library (declared in include/dustin.h).
//
// Every entry point validates its arguments on the host first and returns
// DUSTIN_ERR_INVALID_ARG / DUSTIN_ERR_UNSUPPORTED before touching the HIP
// runtime, then enqueues its kernels on the caller's stream.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "dustin.h"
#include "common.h"
#include "internal.h"
#include <vector>

using namespace dustin;

namespace {

thread_local std::string g_last_error;

dustin_status fail(dustin_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

dustin_status ok() {
    g_last_error.clear();
    return DUSTIN_OK;
}

dustin_status hip_status(hipError_t e, const char *where) {
    if (e == hipSuccess) return ok();
    return fail(DUSTIN_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define CHECK(cond, st, ...)                         \
    do {                                             \
        if (!(cond)) return fail((st), __VA_ARGS__); \
    } while (0)

constexpr int64_t kInt32Max = 2147483647LL;

dustin_status check_kv(const dustin_kv *kv, const char *what, bool need_v) {
    CHECK(kv != nullptr, DUSTIN_ERR_INVALID_ARG, "%s: descriptor is NULL", what);
    CHECK(kv->k != nullptr, DUSTIN_ERR_INVALID_ARG, "%s: k is NULL", what);
    CHECK(!need_v || kv->v != nullptr, DUSTIN_ERR_INVALID_ARG, "%s: v is NULL", what);
    CHECK(kv->dtype == DUSTIN_F32 || kv->dtype == DUSTIN_BF16, DUSTIN_ERR_UNSUPPORTED,
          "%s: dtype %d not supported", what, kv->dtype);
    CHECK(kv->B >= 1 && kv->H_kv >= 1 && kv->N_max >= 1, DUSTIN_ERR_INVALID_ARG,
          "%s: B, H_kv and N_max must be >= 1 (got %d, %d, %d)", what, kv->B, kv->H_kv, kv->N_max);
    CHECK(kv->head_dim == 32 || kv->head_dim == 64 || kv->head_dim == 128, DUSTIN_ERR_UNSUPPORTED,
          "%s: head_dim %d not supported (32, 64, 128)", what, kv->head_dim);
    CHECK(kv->seq_lens != nullptr, DUSTIN_ERR_INVALID_ARG, "%s: seq_lens is NULL", what);
    if (kv->page_size == 0) {
        CHECK((int64_t)kv->B * kv->N_max <= kInt32Max, DUSTIN_ERR_UNSUPPORTED, "%s: B * N_max too large", what);
    } else if (kv->page_size == 16) {
        CHECK(kv->page_table != nullptr, DUSTIN_ERR_INVALID_ARG, "%s: paged cache without page_table", what);
        CHECK(kv->max_pages >= (kv->N_max + 15) / 16, DUSTIN_ERR_INVALID_ARG,
              "%s: max_pages %d < ceil(N_max / 16)", what, kv->max_pages);
        CHECK(kv->num_pages >= 1 && (int64_t)kv->num_pages * 16 <= kInt32Max, DUSTIN_ERR_INVALID_ARG,
              "%s: num_pages %d out of range", what, kv->num_pages);
    } else {
        return fail(DUSTIN_ERR_UNSUPPORTED, "%s: page_size %d not supported (0, 16)", what, kv->page_size);
    }
    return DUSTIN_OK;
}

KvView view_of(const dustin_kv *kv) {
    KvView v{};
    v.k = (const char *)kv->k;
    v.v = (const char *)kv->v;
    v.seq_lens = kv->seq_lens;
    v.page_table = kv->page_size ? kv->page_table : nullptr;
    v.B = kv->B;
    v.Hkv = kv->H_kv;
    v.D = kv->head_dim;
    v.N_max = kv->N_max;
    v.page_size = kv->page_size;
    v.max_pages = kv->max_pages;
    v.num_pages = kv->num_pages;
    v.f32 = kv->dtype == DUSTIN_F32;
    return v;
}

bool same_geometry(const dustin_kv *a, const dustin_kv *b) {
    return a->B == b->B && a->N_max == b->N_max && a->H_kv == b->H_kv && a->head_dim == b->head_dim &&
           a->dtype == b->dtype && a->page_size == b->page_size;
}

float resolve_scale(float scale, int d) { return scale == 0.f ? 1.f / std::sqrt((float)d) : scale; }

dustin_status check_attn_shape(const dustin_kv *kv, int w, int H_q, const char *what) {
    CHECK(w >= 1 && H_q >= 1, DUSTIN_ERR_INVALID_ARG, "%s: w and H_q must be >= 1", what);
    CHECK(H_q % kv->H_kv == 0, DUSTIN_ERR_INVALID_ARG, "%s: H_q %d not a multiple of H_kv %d", what, H_q, kv->H_kv);
    CHECK(w * (H_q / kv->H_kv) <= 64, DUSTIN_ERR_UNSUPPORTED, "%s: w * G = %d exceeds 64", what, w * (H_q / kv->H_kv));

    CHECK((int64_t)kv->B * kv->H_kv <= kAttnCounterSlots, DUSTIN_ERR_UNSUPPORTED,
          "%s: B * H_kv = %lld exceeds %d", what, (long long)kv->B * kv->H_kv, kAttnCounterSlots);
    return DUSTIN_OK;
}

struct WindowLayout {
    AttnPlan plan;
    size_t off_out, off_lse, bytes;
};

size_t window_steps_offset() { return align_up((size_t)kAttnCounterSlots * sizeof(int32_t), 256); }

WindowLayout window_layout(int B, int w, int H_q, int H_kv, int D, int N_max, int esz) {
    WindowLayout L{};
    L.plan = attn_plan(B, w, H_q, H_kv, D, N_max, false);
    size_t off = L.plan.ws_bytes;
    L.off_out = off;
    off = align_up(off + (size_t)B * w * H_q * D * esz, 256);
    L.off_lse = off;
    off = align_up(off + (size_t)B * w * H_q * sizeof(float), 256);
    // the statistics path (window_steps) needs the draft-side scoring
    // workspace, placed after the arrival-counter region so that region stays
    // zero for the attention calls that share the workspace
    const size_t steps = window_steps_offset() + score_plan(B, N_max, 1, H_q, w, 0, H_kv).ws_bytes;
    L.bytes = off > steps ? off : steps;
    return L;
}

// The window attention through the statistics passes (one K read for the
// row normalisers, one for the probabilities, both on MFMA), bfloat16: the
// window steps per pass are at most four (per-step lane sums) and at most 64
// rows per KV head; 0 when the form does not apply.
int window_steps_group(const dustin_kv *kv, int w, int H_q) {
    const int G = H_q / kv->H_kv;
    if (kv->dtype != DUSTIN_BF16 || kv->B > kMaxDraftBatch || G > 64) return 0;
    return std::min(std::min(w, 4), 64 / G);
}

// The statistics form over w window steps whose queries sit at
// q + b * q_bstride + s * q_sstride (elements, [H_q][head_dim] each) and whose
// weights go to A + (b * a_bstride + s * a_sstride) * N_max, in slices of
// window_steps_group steps on the workspace's statistics region.  The
// caller has checked that the form applies; a step stride too large for the
// kernels' 32-bit query offsets returns DUSTIN_ERR_UNSUPPORTED.
dustin_status window_steps_run(const void *q, int64_t q_bstride, int64_t q_sstride, int w, int H_q,
                               const dustin_kv *kv, float scale, float *A, int64_t a_bstride, int64_t a_sstride,
                               char *wsb, hipStream_t stream) {
    const int wg = window_steps_group(kv, w, H_q);
    CHECK(wg > 0, DUSTIN_ERR_UNSUPPORTED, "window_attn: the statistics form does not apply");
    CHECK((int64_t)(wg - 1) * q_sstride + (int64_t)H_q * kv->head_dim < ((int64_t)1 << 29), DUSTIN_ERR_UNSUPPORTED,
          "window_attn: query step stride %lld too large", (long long)q_sstride);
    const size_t esz = 2;
    for (int s0 = 0; s0 < w; s0 += wg) {
        const int g = std::min(wg, w - s0);
        DraftScoreArgs da{};
        da.kv[0] = view_of(kv);
        da.L_d = 1;
        da.H_d = H_q;
        da.gamma = g;
        da.Hkv_d = kv->H_kv;
        da.G_d = H_q / kv->H_kv;
        da.rows = g * da.G_d;
        da.q_draft = (const char *)q + (size_t)s0 * q_sstride * esz;
        da.q_bstride = q_bstride;
        da.q_sstride = q_sstride;
        da.scale_log2 = resolve_scale(scale, kv->head_dim) * kLog2e;
        const ScorePlan sp = score_plan(kv->B, kv->N_max, 1, H_q, g, 0, kv->H_kv);
        char *sws = wsb + window_steps_offset();
        da.stat = (float *)(sws + sp.off_dstat);
        da.lse = (float *)(sws + sp.off_dlse);
        da.nchunk = sp.nchunk;
        da.steps_out = A + (size_t)s0 * a_sstride * kv->N_max;
        da.steps_bstride = (int32_t)a_bstride;
        da.steps_sstride = (int32_t)a_sstride;
        da.steps_scale = 1.f / (float)H_q;
        const hipError_t e = launch_window_steps(da, stream);
        if (e != hipSuccess) return hip_status(e, "window_attn launch");
    }
    return ok();
}

}  // namespace

extern "C" {

const char *dustin_status_string(dustin_status st) {
    switch (st) {
        case DUSTIN_OK: return "DUSTIN_OK";
        case DUSTIN_ERR_INVALID_ARG: return "DUSTIN_ERR_INVALID_ARG";
        case DUSTIN_ERR_UNSUPPORTED: return "DUSTIN_ERR_UNSUPPORTED";
        case DUSTIN_ERR_HIP: return "DUSTIN_ERR_HIP";
    }
    return "DUSTIN_ERR_UNKNOWN";
}

const char *dustin_last_error(void) { return g_last_error.c_str(); }

int32_t dustin_abi_version(void) { return DUSTIN_ABI_VERSION; }

size_t dustin_attn_workspace_bytes(int32_t B, int32_t w, int32_t H_q, int32_t H_kv, int32_t head_dim, int32_t k_or_n) {
    if (B < 1 || w < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || head_dim < 1 || k_or_n < 1) return 0;
    return attn_plan(B, w, H_q, H_kv, head_dim, k_or_n, false).ws_bytes;
}

}  // extern "C"

namespace {
// Checks and kernel arguments shared by dustin_sparse_verify_attn (causal =
// 0), dustin_verify_attn and dustin_verify_attn_append (causal = 1: the w
// window rows after each history are attended causally).  No HIP call.
// Workspace layout of one attention call: arrival counters at the start,
// split partials (m, l, O) at the plan's offsets.
void bind_attn_workspace(AttnArgs &a, const AttnPlan &p, char *wsb) {
    a.counters = (int32_t *)wsb;
    a.part_m = (float *)(wsb + p.off_m);
    a.part_l = (float *)(wsb + p.off_l);
    a.part_o = (float *)(wsb + p.off_o);
}

dustin_status attn_prepare(const char *name, const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                           const int32_t *idx, const int32_t *count, int32_t k, float scale, void *out,
                           float *lse, void *ws, size_t ws_bytes, int causal, AttnArgs &a, AttnPlan &p,
                           bool own_scratch = false) {
    char what[96];
    snprintf(what, sizeof what, "%s kv", name);
    dustin_status st = check_kv(kv, what, true);
    if (st != DUSTIN_OK) return st;
    if ((st = check_attn_shape(kv, w, H_q, name)) != DUSTIN_OK) return st;
    CHECK(q != nullptr && out != nullptr, DUSTIN_ERR_INVALID_ARG, "%s: q and out are required", name);
    if (idx) {
        CHECK(count != nullptr, DUSTIN_ERR_INVALID_ARG, "%s: count is NULL", name);
        CHECK(k >= 1, DUSTIN_ERR_INVALID_ARG, "%s: k must be >= 1 (got %d)", name, k);
    } else {
        CHECK(k == 0, DUSTIN_ERR_INVALID_ARG, "%s: dense form (idx NULL) needs k == 0", name);
    }
    CHECK(std::isfinite(scale), DUSTIN_ERR_INVALID_ARG, "%s: scale is not finite", name);
    const int tokens = (idx ? k : kv->N_max) + (causal ? w : 0);
    p = attn_plan(kv->B, w, H_q, kv->H_kv, kv->head_dim, tokens, kv->dtype == DUSTIN_F32);
    CHECK((int64_t)p.tps * p.splits >= tokens && p.splits < 32768, DUSTIN_ERR_UNSUPPORTED, "%s: too many tokens", name);
    // the allocation-free entry point passes no workspace (own_scratch) and
    // binds its static scratch afterwards
    CHECK(own_scratch || (ws != nullptr && ws_bytes >= p.ws_bytes), DUSTIN_ERR_INVALID_ARG,
          "%s: workspace of %zu bytes needed (got %zu)", name, p.ws_bytes, ws_bytes);
    a = AttnArgs{};
    a.kv = view_of(kv);
    a.q = q;
    a.w = w;
    a.Hq = H_q;
    a.G = H_q / kv->H_kv;
    a.R = w * a.G;
    a.idx = idx;
    a.count = count;
    a.k = idx ? k : 0;
    a.scale_log2 = resolve_scale(scale, kv->head_dim) * kLog2e;
    a.out = out;
    a.lse = lse;
    bind_attn_workspace(a, p, (char *)ws);
    a.splits = p.splits;
    a.tps = p.tps;
    a.rpad = p.rpad;
    a.causal = causal;
    return DUSTIN_OK;
}

dustin_status attn_call(const char *name, const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                        const int32_t *idx, const int32_t *count, int32_t k, float scale, void *out, float *lse,
                        void *ws, size_t ws_bytes, dustin_stream_t stream, int causal) {
    AttnArgs a;
    AttnPlan p;
    dustin_status st = attn_prepare(name, q, w, H_q, kv, idx, count, k, scale, out, lse, ws, ws_bytes, causal, a, p);
    if (st != DUSTIN_OK) return st;
    char what[96];
    snprintf(what, sizeof what, "%s launch", name);
    return hip_status(launch_attn(a, p, (hipStream_t)stream), what);
}

// Target side of the scoring calls: checks the (layer, head) rows and their
// layers and fills the layer views, row tables, query pointer and scale.
dustin_status prep_target(const dustin_kv *target_layers, int32_t L_t, const void *q_hist, const int32_t *sub_heads,
                          int32_t S, int32_t H_t, float scale_target, TargetScoreArgs &a, const dustin_kv *&t0) {
    CHECK(target_layers != nullptr && L_t >= 1, DUSTIN_ERR_INVALID_ARG, "score: target_layers missing");
    CHECK(sub_heads != nullptr && q_hist != nullptr, DUSTIN_ERR_INVALID_ARG, "score: sub_heads / q_hist missing");
    CHECK(S <= kMaxScoreRows, DUSTIN_ERR_UNSUPPORTED, "score: S %d exceeds %d", S, kMaxScoreRows);
    CHECK(H_t >= 1, DUSTIN_ERR_INVALID_ARG, "score: H_t must be >= 1");
    CHECK(L_t <= 64, DUSTIN_ERR_UNSUPPORTED, "score: L_t %d exceeds 64", L_t);
    int view_of_layer[64];
    int n_views = 0;
    int layer_ids[8];
    for (int l = 0; l < L_t; ++l) view_of_layer[l] = -1;
    for (int r = 0; r < S; ++r) {
        const int l = sub_heads[2 * r], h = sub_heads[2 * r + 1];
        CHECK(l >= 0 && l < L_t, DUSTIN_ERR_INVALID_ARG, "score: sub_heads[%d] layer %d out of range", r, l);
        CHECK(h >= 0 && h < H_t, DUSTIN_ERR_INVALID_ARG, "score: sub_heads[%d] head %d out of range", r, h);
        if (view_of_layer[l] < 0) {
            dustin_status st = check_kv(&target_layers[l], "score target layer", false);
            if (st != DUSTIN_OK) return st;
            CHECK(n_views < 8, DUSTIN_ERR_UNSUPPORTED, "score: more than 8 distinct target layers");
            CHECK(H_t % target_layers[l].H_kv == 0, DUSTIN_ERR_INVALID_ARG,
                  "score: H_t %d not a multiple of layer %d H_kv", H_t, l);
            view_of_layer[l] = n_views;
            layer_ids[n_views++] = l;
        }
    }
    t0 = &target_layers[layer_ids[0]];
    for (int i = 1; i < n_views; ++i)
        CHECK(same_geometry(&target_layers[layer_ids[i]], t0), DUSTIN_ERR_INVALID_ARG,
              "score: scored target layers differ in geometry");
    for (int i = 0; i < n_views; ++i) a.kv[i] = view_of(&target_layers[layer_ids[i]]);
    a.n_layers = n_views;
    a.q_hist = q_hist;
    a.S = S;
    for (int r = 0; r < S; ++r) {
        const int l = sub_heads[2 * r], h = sub_heads[2 * r + 1];
        a.row_layer[r] = view_of_layer[l];
        a.row_kvh[r] = h / (H_t / target_layers[l].H_kv);
    }
    a.scale_log2 = resolve_scale(scale_target, a.kv[0].D) * kLog2e;
    return DUSTIN_OK;
}

}  // namespace

extern "C" {

dustin_status dustin_sparse_verify_attn(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                                        const int32_t *idx, const int32_t *count, int32_t k, float scale,
                                        void *out, float *lse, void *ws, size_t ws_bytes,
                                        dustin_stream_t stream) {
    return attn_call("sparse_verify_attn", q, w, H_q, kv, idx, count, k, scale, out, lse, ws, ws_bytes, stream, 0);
}

size_t dustin_verify_attn_workspace_bytes(int32_t B, int32_t w, int32_t H_q, int32_t H_kv, int32_t head_dim,
                                          int32_t k_or_n) {
    if (B < 1 || w < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || head_dim < 1 || k_or_n < 1) return 0;
    return attn_plan(B, w, H_q, H_kv, head_dim, k_or_n + w, false).ws_bytes;
}

dustin_status dustin_verify_attn(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv, const int32_t *idx,
                                 const int32_t *count, int32_t k, float scale, void *out, float *lse, void *ws,
                                 size_t ws_bytes, dustin_stream_t stream) {
    return attn_call("verify_attn", q, w, H_q, kv, idx, count, k, scale, out, lse, ws, ws_bytes, stream, 1);
}

dustin_status dustin_verify_attn_append(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                                        const void *k_win, const void *v_win, const int32_t *idx,
                                        const int32_t *count, int32_t k, float scale, void *out, float *lse,
                                        void *ws, size_t ws_bytes, dustin_stream_t stream) {
    CHECK(k_win != nullptr && v_win != nullptr, DUSTIN_ERR_INVALID_ARG,
          "verify_attn_append: k_win and v_win are required");
    CHECK(kv != nullptr, DUSTIN_ERR_INVALID_ARG, "verify_attn_append: kv is NULL");
    CHECK(((uintptr_t)kv->k | (uintptr_t)kv->v | (uintptr_t)k_win | (uintptr_t)v_win) % 16 == 0,
          DUSTIN_ERR_INVALID_ARG, "verify_attn_append: k, v, k_win and v_win must be 16-byte aligned");
    AttnArgs a;
    AttnPlan p;
    dustin_status st = attn_prepare("verify_attn_append", q, w, H_q, kv, idx, count, k, scale, out, lse, ws,
                                    ws_bytes, 1, a, p);
    if (st != DUSTIN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (kv->dtype == DUSTIN_F32) {   // float32 caches: the append, then the attention
        hipError_t e = launch_append_window(a.kv, k_win, v_win, w, s);
        if (e != hipSuccess) return hip_status(e, "verify_attn_append: append launch");
    } else {
        a.k_win = (const char *)k_win;
        a.v_win = (const char *)v_win;
    }
    return hip_status(launch_attn(a, p, s), "verify_attn_append launch");
}

dustin_status dustin_append_window_kv(const dustin_kv *kv, const void *k_win, const void *v_win, int32_t w,
                                      dustin_stream_t stream) {
    dustin_status st = check_kv(kv, "append_window_kv kv", true);
    if (st != DUSTIN_OK) return st;
    CHECK(k_win != nullptr && v_win != nullptr, DUSTIN_ERR_INVALID_ARG, "append_window_kv: k_win and v_win are required");
    CHECK(w >= 1, DUSTIN_ERR_INVALID_ARG, "append_window_kv: w must be >= 1 (got %d)", w);
    CHECK(((uintptr_t)kv->k | (uintptr_t)kv->v | (uintptr_t)k_win | (uintptr_t)v_win) % 16 == 0,
          DUSTIN_ERR_INVALID_ARG, "append_window_kv: k, v, k_win and v_win must be 16-byte aligned");
    return hip_status(launch_append_window(view_of(kv), k_win, v_win, w, (hipStream_t)stream), "append_window_kv launch");
}

dustin_status dustin_commit_window(int32_t *seq_lens, const int32_t *accepted, int32_t B, int32_t w,
                                   dustin_stream_t stream) {
    CHECK(seq_lens != nullptr && accepted != nullptr, DUSTIN_ERR_INVALID_ARG,
          "commit_window: seq_lens and accepted are required");
    CHECK(B >= 1 && w >= 1, DUSTIN_ERR_INVALID_ARG, "commit_window: B and w must be >= 1");
    return hip_status(launch_commit_window(seq_lens, accepted, B, w, (hipStream_t)stream), "commit_window launch");
}

size_t dustin_window_attn_workspace_bytes(int32_t B, int32_t w, int32_t H_q, int32_t H_kv, int32_t head_dim,
                                          int32_t N_max) {
    if (B < 1 || w < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || head_dim < 1 || N_max < 1) return 0;
    return window_layout(B, w, H_q, H_kv, head_dim, N_max, 4).bytes;
}

dustin_status dustin_window_attn(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv, float scale, float *A,
                                 void *ws, size_t ws_bytes, dustin_stream_t stream) {
    dustin_status st = check_kv(kv, "window_attn kv", false);
    if (st != DUSTIN_OK) return st;
    CHECK(w >= 1 && H_q >= 1, DUSTIN_ERR_INVALID_ARG, "window_attn: w and H_q must be >= 1");
    CHECK(H_q % kv->H_kv == 0, DUSTIN_ERR_INVALID_ARG, "window_attn: H_q %d not a multiple of H_kv %d", H_q,
          kv->H_kv);
    CHECK(w <= 16, DUSTIN_ERR_UNSUPPORTED, "window_attn: w %d exceeds 16", w);
    // the statistics form takes the window in slices; the dense-pass form
    // (float32) has the attention kernel's limits
    if (!window_steps_group(kv, w, H_q) && (st = check_attn_shape(kv, w, H_q, "window_attn")) != DUSTIN_OK)
        return st;
    CHECK(q != nullptr && A != nullptr, DUSTIN_ERR_INVALID_ARG, "window_attn: q and A are required");
    CHECK(std::isfinite(scale), DUSTIN_ERR_INVALID_ARG, "window_attn: scale is not finite");
    // The dense pass needs V only for its (discarded) output; K stands in.
    const WindowLayout L = window_layout(kv->B, w, H_q, kv->H_kv, kv->head_dim, kv->N_max, 4);
    CHECK(ws != nullptr && ws_bytes >= L.bytes, DUSTIN_ERR_INVALID_ARG,
          "window_attn: workspace of %zu bytes needed (got %zu)", L.bytes, ws_bytes);
    char *wsb = (char *)ws;
    if (window_steps_group(kv, w, H_q)) {
        // [B][w][H_q][head_dim] queries, [B][w][N_max] weights
        const int64_t qs = (int64_t)H_q * kv->head_dim;
        return window_steps_run(q, w * qs, qs, w, H_q, kv, scale, A, w, 1, wsb, (hipStream_t)stream);
    }
    AttnArgs a{};
    a.kv = view_of(kv);
    a.kv.v = a.kv.k;
    a.q = q;
    a.w = w;
    a.Hq = H_q;
    a.G = H_q / kv->H_kv;
    a.R = w * a.G;
    a.idx = nullptr;
    a.count = nullptr;
    a.k = 0;
    const float sc = resolve_scale(scale, kv->head_dim);
    a.scale_log2 = sc * kLog2e;
    a.out = wsb + L.off_out;
    a.lse = (float *)(wsb + L.off_lse);
    a.counters = (int32_t *)wsb;
    a.part_m = (float *)(wsb + L.plan.off_m);
    a.part_l = (float *)(wsb + L.plan.off_l);
    a.part_o = (float *)(wsb + L.plan.off_o);
    a.splits = L.plan.splits;
    a.tps = L.plan.tps;
    a.rpad = L.plan.rpad;
    hipError_t e = launch_attn(a, L.plan, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "window_attn dense pass");
    WindowArgs wa{};
    wa.kv = view_of(kv);
    wa.q = q;
    wa.w = w;
    wa.Hq = H_q;
    wa.G = a.G;
    wa.scale_log2 = a.scale_log2;
    wa.lse = a.lse;
    wa.A = A;
    return hip_status(launch_window_probs(wa, (hipStream_t)stream), "window_attn probabilities");
}

dustin_status dustin_arr(const float *A, const int32_t *seq_lens, int32_t B, int32_t w, int32_t N_max,
                         const int32_t *idx, const int32_t *count, int32_t k, float *arr_step,
                         float *arr_window, dustin_stream_t stream) {
    CHECK(A && seq_lens && idx && count, DUSTIN_ERR_INVALID_ARG, "arr: A, seq_lens, idx and count are required");
    CHECK(B >= 1 && w >= 1 && N_max >= 1 && k >= 1, DUSTIN_ERR_INVALID_ARG, "arr: B, w, N_max and k must be >= 1");
    CHECK(w <= 64, DUSTIN_ERR_UNSUPPORTED, "arr: w %d exceeds 64", w);
    ArrArgs a{A, seq_lens, B, w, N_max, k, idx, count, arr_step, arr_window};
    if (!arr_step && !arr_window) return ok();
    return hip_status(launch_arr(a, (hipStream_t)stream), "arr launch");
}

size_t dustin_topk_workspace_bytes(int32_t B, int32_t N_max, int32_t k) {
    if (B < 1 || N_max < 1 || k < 1) return 0;
    return topk_plan(B, N_max, k).ws_bytes;
}

dustin_status dustin_topk(const float *s_draft, const float *s_target, const int32_t *seq_lens, int32_t B,
                          int32_t N_max, int32_t k, int32_t m, int32_t n_sink, int32_t n_window, int32_t *idx,
                          int32_t *count, int8_t *tier, void *ws, size_t ws_bytes, dustin_stream_t stream) {
    CHECK(s_draft || s_target, DUSTIN_ERR_INVALID_ARG, "topk: at least one score vector is required");
    CHECK(seq_lens && idx && count, DUSTIN_ERR_INVALID_ARG, "topk: seq_lens, idx and count are required");
    CHECK(B >= 1 && N_max >= 1, DUSTIN_ERR_INVALID_ARG, "topk: B and N_max must be >= 1");
    CHECK(k >= 1, DUSTIN_ERR_INVALID_ARG, "topk: k must be >= 1 (got %d)", k);
    CHECK(m >= 0 && n_sink >= 0 && n_window >= 0, DUSTIN_ERR_INVALID_ARG, "topk: m, n_sink, n_window must be >= 0");
    CHECK((int64_t)n_sink + n_window <= k, DUSTIN_ERR_INVALID_ARG,
          "topk: n_sink + n_window = %d exceeds k = %d", n_sink + n_window, k);
    CHECK((int64_t)B * N_max <= kInt32Max, DUSTIN_ERR_UNSUPPORTED, "topk: B * N_max too large");
    const TopkPlan p = topk_plan(B, N_max, k);
    CHECK(ws != nullptr && ws_bytes >= p.ws_bytes, DUSTIN_ERR_INVALID_ARG,
          "topk: workspace of %zu bytes needed (got %zu)", p.ws_bytes, ws_bytes);
    TopkArgs a{};
    a.s_draft = s_draft;
    a.s_target = s_target;
    a.seq_lens = seq_lens;
    a.B = B;
    a.N_max = N_max;
    a.k = k;
    a.m = m;
    a.n_sink = n_sink;
    a.n_window = n_window;
    a.idx = idx;
    a.count = count;
    a.tier = tier;
    a.flag = (uint8_t *)ws + p.off_flag;
    return hip_status(launch_topk(a, (hipStream_t)stream), "topk launch");
}

size_t dustin_score_workspace_bytes(int32_t B, int32_t N_max, int32_t L_d, int32_t H_d, int32_t gamma, int32_t S) {
    if (B < 1 || N_max < 1 || L_d < 0 || H_d < 0 || gamma < 0 || S < 0) return 0;
    return score_plan(B, N_max, L_d, H_d, gamma, S, 1).ws_bytes;
}

}  // extern "C"

namespace {
// Checks of the draft side of a scoring call; sets the draft KV head count
// and the query heads per KV head.
dustin_status prep_draft(const dustin_kv *draft_layers, int32_t L_d, const void *q_draft, int32_t H_d, int32_t gamma,
                         int &Hkv_d, int &G_d) {
    CHECK(draft_layers != nullptr, DUSTIN_ERR_INVALID_ARG, "score: draft_layers is NULL");
    CHECK(L_d <= kMaxDraftLayers, DUSTIN_ERR_UNSUPPORTED, "score: L_d %d exceeds %d", L_d, kMaxDraftLayers);
    CHECK(draft_layers[0].B <= kMaxDraftBatch, DUSTIN_ERR_UNSUPPORTED, "score: B %d exceeds %d on the draft side",
          draft_layers[0].B, kMaxDraftBatch);
    for (int l = 0; l < L_d; ++l) {
        dustin_status st = check_kv(&draft_layers[l], "score draft layer", false);
        if (st != DUSTIN_OK) return st;
        CHECK(same_geometry(&draft_layers[l], &draft_layers[0]), DUSTIN_ERR_INVALID_ARG,
              "score: draft layer %d differs in geometry from layer 0", l);
    }
    const dustin_kv *ref = &draft_layers[0];
    CHECK(q_draft != nullptr, DUSTIN_ERR_INVALID_ARG, "score: q_draft is NULL");
    CHECK(H_d >= 1 && gamma >= 1, DUSTIN_ERR_INVALID_ARG, "score: H_d and gamma must be >= 1");
    Hkv_d = ref->H_kv;
    CHECK(H_d % Hkv_d == 0, DUSTIN_ERR_INVALID_ARG, "score: H_d %d not a multiple of draft H_kv %d", H_d, Hkv_d);
    G_d = H_d / Hkv_d;
    CHECK(gamma * G_d <= 64, DUSTIN_ERR_UNSUPPORTED, "score: gamma * G_d = %d exceeds 64", gamma * G_d);
    if (ref->dtype == DUSTIN_F32) {
        CHECK(L_d <= 8 && (int64_t)L_d * H_d * gamma <= kMaxScoreQoff &&
                  (int64_t)L_d * Hkv_d * ((gamma * G_d + 7) / 8) <= kMaxScoreRows,
              DUSTIN_ERR_UNSUPPORTED, "score: float32 draft larger than the library supports");
    }
    return ok();
}

DraftScoreArgs draft_args(const dustin_kv *draft_layers, int32_t L_d, const void *q_draft, int32_t H_d,
                          int32_t gamma, int Hkv_d, int G_d, float scale_draft, const ScorePlan &p, char *wsb) {
    DraftScoreArgs a{};
    for (int l = 0; l < L_d; ++l) a.kv[l] = view_of(&draft_layers[l]);
    a.L_d = L_d;
    a.H_d = H_d;
    a.gamma = gamma;
    a.Hkv_d = Hkv_d;
    a.G_d = G_d;
    a.rows = gamma * G_d;
    a.q_draft = q_draft;
    a.scale_log2 = resolve_scale(scale_draft, a.kv[0].D) * kLog2e;
    a.stat = (float *)(wsb + p.off_dstat);
    a.lse = (float *)(wsb + p.off_dlse);
    a.nchunk = p.nchunk;
    a.part = (float *)(wsb + p.off_dpart);
    a.acc_groups = p.acc_groups;
    return a;
}
}  // namespace

extern "C" {

dustin_status dustin_score(const dustin_kv *draft_layers, int32_t L_d, const void *q_draft, int32_t H_d,
                           int32_t gamma, const dustin_kv *target_layers, int32_t L_t, const void *q_hist,
                           const int32_t *sub_heads, int32_t S, int32_t H_t, float scale_draft,
                           float scale_target, const float *draft_lse, float *s_draft, float *s_target, void *ws,
                           size_t ws_bytes, dustin_stream_t stream) {
    const bool do_draft = s_draft != nullptr && L_d > 0;
    const bool do_target = s_target != nullptr && S > 0;
    CHECK(L_d >= 0 && S >= 0 && L_t >= 0, DUSTIN_ERR_INVALID_ARG, "score: negative count");
    CHECK(std::isfinite(scale_draft) && std::isfinite(scale_target), DUSTIN_ERR_INVALID_ARG,
          "score: scale is not finite");
    const dustin_kv *ref = nullptr;
    int Hkv_d = 1;
    int G_d = 1;
    if (do_draft) {
        dustin_status st = prep_draft(draft_layers, L_d, q_draft, H_d, gamma, Hkv_d, G_d);
        if (st != DUSTIN_OK) return st;
        ref = &draft_layers[0];
    }
    TargetScoreArgs ta{};
    if (do_target) {
        const dustin_kv *t0 = nullptr;
        dustin_status st = prep_target(target_layers, L_t, q_hist, sub_heads, S, H_t, scale_target, ta, t0);
        if (st != DUSTIN_OK) return st;
        if (ref) {
            CHECK(t0->B == ref->B && t0->N_max == ref->N_max, DUSTIN_ERR_INVALID_ARG,
                  "score: draft and target describe different batches");
        } else {
            ref = t0;
        }
    }
    if (!do_draft && !do_target) return ok();
    const ScorePlan p = score_plan(ref->B, ref->N_max, do_draft ? L_d : 0, H_d, gamma, do_target ? S : 0, Hkv_d);
    CHECK(ws != nullptr && ws_bytes >= p.ws_bytes, DUSTIN_ERR_INVALID_ARG,
          "score: workspace of %zu bytes needed (got %zu)", p.ws_bytes, ws_bytes);
    char *wsb = (char *)ws;
    hipStream_t s = (hipStream_t)stream;
    if (do_target) {
        ta.s_target = s_target;
        ta.logit = (float *)(wsb + p.off_tlogit);
        ta.stat = (float *)(wsb + p.off_tstat);
        ta.lse = (float *)(wsb + p.off_tlse);
        ta.nchunk = p.nchunk;
        hipError_t e = launch_target_score(ta, s);
        if (e != hipSuccess) return hip_status(e, "score target launch");
    }
    if (do_draft) {
        DraftScoreArgs a = draft_args(draft_layers, L_d, q_draft, H_d, gamma, Hkv_d, G_d, scale_draft, p, wsb);
        a.s_draft = s_draft;
        a.lse_in = draft_lse;
        hipError_t e = launch_draft_score(a, s);
        if (e != hipSuccess) return hip_status(e, "score draft launch");
    }
    return ok();
}

dustin_status dustin_draft_row_lse(const dustin_kv *draft_layers, int32_t L_d, const void *q_draft, int32_t H_d,
                                   int32_t gamma, float scale_draft, float *lse_out, void *ws, size_t ws_bytes,
                                   dustin_stream_t stream) {
    CHECK(L_d >= 1, DUSTIN_ERR_INVALID_ARG, "draft_row_lse: L_d must be >= 1");
    CHECK(lse_out != nullptr, DUSTIN_ERR_INVALID_ARG, "draft_row_lse: lse_out is NULL");
    CHECK(std::isfinite(scale_draft), DUSTIN_ERR_INVALID_ARG, "draft_row_lse: scale is not finite");
    int Hkv_d = 1, G_d = 1;
    dustin_status st = prep_draft(draft_layers, L_d, q_draft, H_d, gamma, Hkv_d, G_d);
    if (st != DUSTIN_OK) return st;
    const dustin_kv *ref = &draft_layers[0];
    const ScorePlan p = score_plan(ref->B, ref->N_max, L_d, H_d, gamma, 0, Hkv_d);
    CHECK(ws != nullptr && ws_bytes >= p.ws_bytes, DUSTIN_ERR_INVALID_ARG,
          "draft_row_lse: workspace of %zu bytes needed (got %zu)", p.ws_bytes, ws_bytes);
    DraftScoreArgs a = draft_args(draft_layers, L_d, q_draft, H_d, gamma, Hkv_d, G_d, scale_draft, p, (char *)ws);
    a.lse_out = lse_out;
    return hip_status(launch_draft_score(a, (hipStream_t)stream), "draft_row_lse launch");
}

}  // extern "C"

namespace {
// Sweep workspace: the window-attention workspace first (its arrival
// counters at offset 0), then A of the window [B][w][N], Abar [B][N], the
// past queries' A [P][B][N], one index set [B][k_max] with its counts, and
// the select workspace.
struct SweepLayout {
    size_t attn_bytes, off_awin, off_abar, off_apast, off_idx, off_cnt, off_topk, bytes;
};

SweepLayout sweep_layout(int B, int w, int P, int H_q, int H_kv, int D, int N, int k_max) {
    SweepLayout L{};
    const size_t a1 = window_layout(B, w, H_q, H_kv, D, N, 4).bytes;
    // the past queries: one step each (dense-pass form) or slices of up to
    // four steps (statistics form)
    const size_t a2 = window_layout(B, std::min(std::max(P, 1), 4), H_q, H_kv, D, N, 4).bytes;
    L.attn_bytes = a1 > a2 ? a1 : a2;
    size_t off = align_up(L.attn_bytes, 256);
    L.off_awin = off;
    off = align_up(off + (size_t)B * w * N * sizeof(float), 256);
    L.off_abar = off;
    off = align_up(off + (size_t)B * N * sizeof(float), 256);
    L.off_apast = off;
    off = align_up(off + (size_t)P * B * N * sizeof(float), 256);
    L.off_idx = off;
    off = align_up(off + (size_t)B * k_max * sizeof(int32_t), 256);
    L.off_cnt = off;
    off = align_up(off + (size_t)B * sizeof(int32_t), 256);
    L.off_topk = off;
    off = align_up(off + topk_plan(B, N, k_max).ws_bytes, 256);
    L.bytes = off;
    return L;
}
}  // namespace

extern "C" {

dustin_status dustin_window_mean(const float *A, int32_t B, int32_t w, int32_t N_max, float *Abar,
                                 dustin_stream_t stream) {
    CHECK(A != nullptr && Abar != nullptr, DUSTIN_ERR_INVALID_ARG, "window_mean: A and Abar are required");
    CHECK(B >= 1 && w >= 1 && N_max >= 1, DUSTIN_ERR_INVALID_ARG, "window_mean: B, w and N_max must be >= 1");
    return hip_status(launch_window_mean(A, B, w, N_max, Abar, (hipStream_t)stream), "window_mean launch");
}

size_t dustin_policy_sweep_workspace_bytes(int32_t B, int32_t w, int32_t n_past, int32_t H_q, int32_t H_kv,
                                           int32_t head_dim, int32_t N_max, int32_t k_max) {
    if (B < 1 || w < 1 || n_past < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv || head_dim < 1 || N_max < 1 || k_max < 1)
        return 0;
    return sweep_layout(B, w, n_past, H_q, H_kv, head_dim, N_max, k_max).bytes;
}

dustin_status dustin_policy_sweep(const void *q_window, int32_t w, const void *q_past, int32_t n_past, int32_t H_q,
                                  const dustin_kv *kv, const float *s_draft, const float *s_target,
                                  const int32_t *ks, const int32_t *m_hybrid, int32_t nk, int32_t n_sink,
                                  int32_t n_window, float scale, float *arr, void *ws, size_t ws_bytes,
                                  dustin_stream_t stream) {
    dustin_status st = check_kv(kv, "policy_sweep kv", false);
    if (st != DUSTIN_OK) return st;
    if ((st = check_attn_shape(kv, w, H_q, "policy_sweep")) != DUSTIN_OK) return st;
    CHECK(w <= 16, DUSTIN_ERR_UNSUPPORTED, "policy_sweep: w %d exceeds 16", w);
    CHECK(n_past >= 0 && n_past <= 64, DUSTIN_ERR_UNSUPPORTED, "policy_sweep: n_past %d outside [0, 64]", n_past);
    CHECK(q_window != nullptr && (n_past == 0 || q_past != nullptr), DUSTIN_ERR_INVALID_ARG,
          "policy_sweep: q_window (and q_past when n_past > 0) are required");
    CHECK(s_draft != nullptr && s_target != nullptr && arr != nullptr, DUSTIN_ERR_INVALID_ARG,
          "policy_sweep: s_draft, s_target and arr are required");
    CHECK(ks != nullptr && m_hybrid != nullptr && nk >= 1, DUSTIN_ERR_INVALID_ARG,
          "policy_sweep: ks, m_hybrid (host arrays) and nk >= 1 are required");
    CHECK(n_sink >= 0 && n_window >= 0, DUSTIN_ERR_INVALID_ARG, "policy_sweep: n_sink and n_window must be >= 0");
    CHECK(std::isfinite(scale), DUSTIN_ERR_INVALID_ARG, "policy_sweep: scale is not finite");
    int k_max = 1;
    for (int i = 0; i < nk; ++i) {
        CHECK(ks[i] >= 1 && (int64_t)n_sink + n_window <= ks[i], DUSTIN_ERR_INVALID_ARG,
              "policy_sweep: ks[%d] = %d must be >= 1 and >= n_sink + n_window", i, ks[i]);
        CHECK(m_hybrid[i] >= 0 && m_hybrid[i] <= ks[i], DUSTIN_ERR_INVALID_ARG,
              "policy_sweep: m_hybrid[%d] = %d outside [0, k]", i, m_hybrid[i]);
        if (ks[i] > k_max) k_max = ks[i];
    }
    const int B = kv->B, N = kv->N_max;
    const SweepLayout L = sweep_layout(B, w, n_past, H_q, kv->H_kv, kv->head_dim, N, k_max);
    CHECK(ws != nullptr && ws_bytes >= L.bytes, DUSTIN_ERR_INVALID_ARG,
          "policy_sweep: workspace of %zu bytes needed (got %zu)", L.bytes, ws_bytes);
    char *wsb = (char *)ws;
    float *Awin = (float *)(wsb + L.off_awin);
    float *Abar = (float *)(wsb + L.off_abar);
    float *Apast = (float *)(wsb + L.off_apast);
    int32_t *idx = (int32_t *)(wsb + L.off_idx);
    int32_t *cnt = (int32_t *)(wsb + L.off_cnt);
    void *tws = wsb + L.off_topk;
    const size_t tbytes = L.bytes - L.off_topk;
    // ground truth: A of the window (Eq. 1) and its mean (Eq. 3)
    if ((st = dustin_window_attn(q_window, w, H_q, kv, scale, Awin, wsb, L.attn_bytes, stream)) != DUSTIN_OK)
        return st;
    {
        const hipError_t e = launch_window_mean(Awin, B, w, N, Abar, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e, "policy_sweep window mean");
    }
    // A_{i-delta,.} of each past query: the past queries [n_past][B][H_q][d]
    // are the steps of one window (step-major), so the statistics form reads
    // K twice per four of them; otherwise one one-step window each
    const size_t esz = kv->dtype == DUSTIN_F32 ? 4 : 2;
    const size_t qstride = (size_t)B * H_q * kv->head_dim * esz;
    if (n_past > 0 && window_steps_group(kv, n_past, H_q)) {
        if ((st = window_steps_run(q_past, (int64_t)H_q * kv->head_dim, (int64_t)B * H_q * kv->head_dim, n_past, H_q,
                                   kv, scale, Apast, 1, B, wsb, (hipStream_t)stream)) != DUSTIN_OK)
            return st;
    } else {
        for (int p = 0; p < n_past; ++p)
            if ((st = dustin_window_attn((const char *)q_past + p * qstride, 1, H_q, kv, scale,
                                         Apast + (size_t)p * B * N, wsb, L.attn_bytes, stream)) != DUSTIN_OK)
                return st;
    }
    auto eval = [&](const float *sd, const float *stg, int k, int m, int ns, int nw, int row, int ki) {
        dustin_status e = dustin_topk(sd, stg, kv->seq_lens, B, N, k, m, ns, nw, idx, cnt, nullptr, tws, tbytes, stream);
        if (e != DUSTIN_OK) return e;
        return dustin_arr(Awin, kv->seq_lens, B, w, N, idx, cnt, k, nullptr, arr + ((size_t)row * nk + ki) * B, stream);
    };
    for (int ki = 0; ki < nk; ++ki) {
        const int k = ks[ki];
        if ((st = eval(nullptr, Abar, k, 0, 0, 0, 0, ki)) != DUSTIN_OK) return st;
        for (int p = 0; p < n_past; ++p)
            if ((st = eval(nullptr, Apast + (size_t)p * B * N, k, 0, 0, 0, 1 + p, ki)) != DUSTIN_OK) return st;
        if ((st = eval(s_draft, nullptr, k, k, 0, 0, n_past + 1, ki)) != DUSTIN_OK) return st;
        const int ms[3] = {0, k - n_sink - n_window, m_hybrid[ki]};
        for (int r = 0; r < 3; ++r)
            if ((st = eval(s_draft, s_target, k, ms[r], n_sink, n_window, n_past + 2 + r, ki)) != DUSTIN_OK) return st;
    }
    return ok();
}

}  // extern "C"

extern "C" {

dustin_status dustin_page_bounds(const dustin_kv *kv, void *kmin, void *kmax, dustin_stream_t stream) {
    dustin_status st = check_kv(kv, "page_bounds kv", false);
    if (st != DUSTIN_OK) return st;
    CHECK(kmin != nullptr && kmax != nullptr, DUSTIN_ERR_INVALID_ARG, "page_bounds: kmin and kmax are required");
    CHECK(kv->H_kv * kv->head_dim <= kPageMaxRow, DUSTIN_ERR_UNSUPPORTED,
          "page_bounds: H_kv * head_dim = %d exceeds %d", kv->H_kv * kv->head_dim, kPageMaxRow);
    CHECK(((uintptr_t)kmin | (uintptr_t)kmax | (uintptr_t)kv->k) % 16 == 0, DUSTIN_ERR_INVALID_ARG,
          "page_bounds: k, kmin and kmax must be 16-byte aligned");
    PageArgs a{};
    a.kv = view_of(kv);
    a.kmin = kmin;
    a.kmax = kmax;
    a.npages = (kv->N_max + 15) / 16;
    return hip_status(launch_page_bounds(a, (hipStream_t)stream), "page_bounds launch");
}

size_t dustin_page_scores_workspace_bytes(int32_t B, int32_t H_kv, int32_t head_dim) {
    if (B < 1 || H_kv < 1 || head_dim < 1) return 0;
    return align_up((size_t)B * 2 * H_kv * head_dim * sizeof(float), 256);
}

dustin_status dustin_page_scores(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv, const void *kmin,
                                 const void *kmax, float scale, float *scores, void *ws, size_t ws_bytes,
                                 dustin_stream_t stream) {
    dustin_status st = check_kv(kv, "page_scores kv", false);
    if (st != DUSTIN_OK) return st;
    CHECK(q != nullptr && kmin != nullptr && kmax != nullptr && scores != nullptr, DUSTIN_ERR_INVALID_ARG,
          "page_scores: q, kmin, kmax and scores are required");
    CHECK(w >= 1 && H_q >= 1 && H_q % kv->H_kv == 0, DUSTIN_ERR_INVALID_ARG,
          "page_scores: w >= 1 and H_q a multiple of H_kv are required");
    CHECK(kv->H_kv * kv->head_dim <= kPageMaxRow, DUSTIN_ERR_UNSUPPORTED,
          "page_scores: H_kv * head_dim = %d exceeds %d", kv->H_kv * kv->head_dim, kPageMaxRow);
    CHECK(((uintptr_t)q | (uintptr_t)kmin | (uintptr_t)kmax) % 16 == 0, DUSTIN_ERR_INVALID_ARG,
          "page_scores: q, kmin and kmax must be 16-byte aligned");
    CHECK(std::isfinite(scale), DUSTIN_ERR_INVALID_ARG, "page_scores: scale is not finite");
    CHECK((int64_t)((kv->N_max + 15) / 16) * kv->H_kv * kv->head_dim * (kv->dtype == DUSTIN_F32 ? 4 : 2) <= kInt32Max,
          DUSTIN_ERR_UNSUPPORTED, "page_scores: one sequence's bounds exceed 2 GiB");
    const size_t need = dustin_page_scores_workspace_bytes(kv->B, kv->H_kv, kv->head_dim);
    CHECK(ws != nullptr && ws_bytes >= need && (uintptr_t)ws % 16 == 0, DUSTIN_ERR_INVALID_ARG,
          "page_scores: 16-byte aligned workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    PageArgs a{};
    a.pm = (float *)ws;
    a.kv = view_of(kv);
    a.q = q;
    a.w = w;
    a.Hq = H_q;
    a.kmin = const_cast<void *>(kmin);
    a.kmax = const_cast<void *>(kmax);
    a.npages = (kv->N_max + 15) / 16;
    a.scale = resolve_scale(scale, kv->head_dim);
    a.scores = scores;
    return hip_status(launch_page_scores(a, (hipStream_t)stream), "page_scores launch");
}

}  // extern "C"

namespace {
// Candidate-evaluation workspace: the unit index list, the materialised
// candidate rows (when a side adds units to a base or picks units by index),
// the index sets and counts of all C * B rows, and the select kernels' flag
// array when the general select kernel runs (N_max > 131072).
struct CandLayout {
    size_t off_ids, off_rows, off_idx, off_cnt, off_flag, bytes;
};

CandLayout cand_layout(int C, int B, int N_max, int k, bool materialize) {
    CandLayout L{};
    const size_t rows = (size_t)C * B;
    size_t off = 0;
    L.off_ids = off;
    off = align_up(off + (size_t)C * sizeof(int32_t), 256);
    L.off_rows = off;
    if (materialize) off = align_up(off + rows * N_max * sizeof(float), 256);
    L.off_idx = off;
    off = align_up(off + rows * k * sizeof(int32_t), 256);
    L.off_cnt = off;
    off = align_up(off + rows * sizeof(int32_t), 256);
    L.off_flag = off;
    off = align_up(off + topk_plan((int)rows, N_max, k).ws_bytes, 256);   // shared by the candidates' launches
    L.bytes = off;
    return L;
}

struct CandSide {
    const float *base, *units;
};

// Evaluates C candidates (arguments already checked): per side, either a base
// vector shared by every candidate, units (one per candidate, optionally by
// index), or both (materialised sums).  m_cand (host, nullable) gives each
// candidate its own m.
dustin_status cand_run(CandSide d, CandSide t, int U, const int32_t *unit_ids, int C, const int32_t *m_cand,
                       const int32_t *seq_lens, int B, int N_max, const float *abar, int k, int m, int n_sink,
                       int n_window, float *arr, float *arr_mean, char *ws, hipStream_t s) {
    (void)U;
    const bool has_units = d.units || t.units;
    const bool mat = has_units && (unit_ids != nullptr || (d.units ? d.base : t.base) != nullptr);
    const CandLayout L = cand_layout(C, B, N_max, k, mat);
    const int32_t *ids_dev = nullptr;
    if (has_units && unit_ids) {
        hipError_t e = hipMemcpyAsync(ws + L.off_ids, unit_ids, (size_t)C * sizeof(int32_t), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, "candidate ids copy");
        ids_dev = (const int32_t *)(ws + L.off_ids);
    }
    // per side: the pointer the select kernels read and its row modulus
    const float *pd = nullptr, *pt = nullptr;
    int md = 0, mt = 0;
    auto place = [&](CandSide c, const float *&ptr, int &mod) -> hipError_t {
        if (!c.base && !c.units) return hipSuccess;
        if (!c.units) {
            ptr = c.base;
            mod = B;
            return hipSuccess;
        }
        if (mat) {
            float *rows = (float *)(ws + L.off_rows);
            if (ids_dev) {
                hipError_t e = launch_build_rows(c.base, c.units, ids_dev, C, B, N_max, rows, s);
                if (e != hipSuccess) return e;
            } else {
                // identity ids: candidate c is unit c
                hipError_t e = hipSuccess;
                for (int cc = 0; cc < C && e == hipSuccess; ++cc) {
                    float *dst = rows + (size_t)cc * B * N_max;
                    e = launch_accumulate(dst, c.base, (int64_t)B * N_max, true, s);
                    if (e == hipSuccess) e = launch_accumulate(dst, c.units + (size_t)cc * B * N_max, (int64_t)B * N_max, false, s);
                }
                if (e != hipSuccess) return e;
            }
            ptr = rows;
        } else {
            ptr = c.units;   // rows c * B + b are contiguous
        }
        mod = 0;
        return hipSuccess;
    };
    hipError_t e = place(d, pd, md);
    if (e == hipSuccess) e = place(t, pt, mt);
    if (e != hipSuccess) return hip_status(e, "candidate rows");
    int32_t *idx = (int32_t *)(ws + L.off_idx);
    int32_t *cnt = (int32_t *)(ws + L.off_cnt);
    TopkArgs a{};
    a.seq_lens = seq_lens;
    a.N_max = N_max;
    a.k = k;
    a.n_sink = n_sink;
    a.n_window = n_window;
    a.tier = nullptr;
    a.flag = (uint8_t *)(ws + L.off_flag);
    a.len_mod = B;
    if (!m_cand) {
        a.s_draft = pd;
        a.s_target = pt;
        a.d_mod = md;
        a.t_mod = mt;
        a.B = C * B;
        a.m = m;
        a.idx = idx;
        a.count = cnt;
        e = launch_topk(a, s);
    } else {
        for (int c = 0; c < C && e == hipSuccess; ++c) {
            const size_t off = (size_t)c * B;
            a.s_draft = pd ? (md ? pd : pd + off * N_max) : nullptr;
            a.s_target = pt ? (mt ? pt : pt + off * N_max) : nullptr;
            a.d_mod = md;
            a.t_mod = mt;
            a.B = B;
            a.m = m_cand[c];
            a.idx = idx + off * k;
            a.count = cnt + off;
            a.flag = (uint8_t *)(ws + L.off_flag);   // launches in stream order share the select workspace
            e = launch_topk(a, s);
        }
    }
    if (e == hipSuccess) e = launch_gather_sum(abar, idx, cnt, C * B, B, N_max, k, arr, s);
    if (e == hipSuccess && arr_mean) e = launch_batch_mean(arr, C, B, arr_mean, s);
    return hip_status(e, "candidate evaluation");
}

dustin_status cand_check(const float *s_draft, const float *draft_units, const float *s_target,
                         const float *target_units, int32_t U, const int32_t *unit_ids, int32_t C,
                         const int32_t *m_cand, const int32_t *seq_lens, int32_t B, int32_t N_max, const float *abar,
                         int32_t k, int32_t m, int32_t n_sink, int32_t n_window, const char *name) {
    CHECK(s_draft || draft_units || s_target || target_units, DUSTIN_ERR_INVALID_ARG,
          "%s: at least one score side is required", name);
    CHECK(!(draft_units && target_units), DUSTIN_ERR_INVALID_ARG, "%s: units on one side only", name);
    CHECK(seq_lens && abar, DUSTIN_ERR_INVALID_ARG, "%s: seq_lens and abar are required", name);
    CHECK(C >= 1 && B >= 1 && N_max >= 1 && k >= 1, DUSTIN_ERR_INVALID_ARG, "%s: C, B, N_max, k must be >= 1", name);
    CHECK(m >= 0 && n_sink >= 0 && n_window >= 0 && (int64_t)n_sink + n_window <= k, DUSTIN_ERR_INVALID_ARG,
          "%s: need m, n_sink, n_window >= 0 and n_sink + n_window <= k", name);
    CHECK((int64_t)C * B <= (1 << 24) && (int64_t)C * B * N_max <= ((int64_t)1 << 40), DUSTIN_ERR_UNSUPPORTED,
          "%s: C * B = %lld rows too many", name, (long long)C * B);
    if (draft_units || target_units) {
        CHECK(U >= 1, DUSTIN_ERR_INVALID_ARG, "%s: U must be >= 1", name);
        if (unit_ids) {
            for (int c = 0; c < C; ++c)
                CHECK(unit_ids[c] >= 0 && unit_ids[c] < U, DUSTIN_ERR_INVALID_ARG, "%s: unit_ids[%d] = %d out of [0, %d)",
                      name, c, unit_ids[c], U);
        } else {
            CHECK(C <= U, DUSTIN_ERR_INVALID_ARG, "%s: C = %d exceeds U = %d without unit_ids", name, C, U);
        }
    }
    if (m_cand)
        for (int c = 0; c < C; ++c)
            CHECK(m_cand[c] >= 0, DUSTIN_ERR_INVALID_ARG, "%s: m_cand[%d] < 0", name, c);
    return DUSTIN_OK;
}
}  // namespace

extern "C" {

size_t dustin_head_scores_workspace_bytes(int32_t B, int32_t N_max, int32_t S) {
    if (B < 1 || N_max < 1 || S < 1) return 0;
    return score_plan(B, N_max, 0, 0, 0, S, 1).ws_bytes;
}

dustin_status dustin_head_scores(const dustin_kv *target_layers, int32_t L_t, const void *q_hist,
                                 const int32_t *sub_heads, int32_t S, int32_t H_t, float scale, float *out, void *ws,
                                 size_t ws_bytes, dustin_stream_t stream) {
    CHECK(S >= 1, DUSTIN_ERR_INVALID_ARG, "head_scores: S must be >= 1");
    CHECK(out != nullptr, DUSTIN_ERR_INVALID_ARG, "head_scores: out is required");
    CHECK(std::isfinite(scale), DUSTIN_ERR_INVALID_ARG, "head_scores: scale is not finite");
    TargetScoreArgs a{};
    const dustin_kv *t0 = nullptr;
    dustin_status st = prep_target(target_layers, L_t, q_hist, sub_heads, S, H_t, scale, a, t0);
    if (st != DUSTIN_OK) return st;
    const ScorePlan p = score_plan(t0->B, t0->N_max, 0, 0, 0, S, 1);
    CHECK(ws != nullptr && ws_bytes >= p.ws_bytes, DUSTIN_ERR_INVALID_ARG,
          "head_scores: workspace of %zu bytes needed (got %zu)", p.ws_bytes, ws_bytes);
    char *wsb = (char *)ws;
    a.s_target = nullptr;
    a.rows_out = out;
    a.logit = (float *)(wsb + p.off_tlogit);
    a.stat = (float *)(wsb + p.off_tstat);
    a.lse = (float *)(wsb + p.off_tlse);
    a.nchunk = p.nchunk;
    return hip_status(launch_target_score(a, (hipStream_t)stream), "head_scores launch");
}

size_t dustin_candidate_arr_workspace_bytes(int32_t C, int32_t B, int32_t N_max, int32_t k, int32_t materialize) {
    if (C < 1 || B < 1 || N_max < 1 || k < 1) return 0;
    return cand_layout(C, B, N_max, k, materialize != 0).bytes;
}

dustin_status dustin_candidate_arr(const float *s_draft, const float *draft_units, const float *s_target,
                                   const float *target_units, int32_t U, const int32_t *unit_ids, int32_t C,
                                   const int32_t *m_cand, const int32_t *seq_lens, int32_t B, int32_t N_max,
                                   const float *abar, int32_t k, int32_t m, int32_t n_sink, int32_t n_window,
                                   float *arr, float *arr_mean, void *ws, size_t ws_bytes, dustin_stream_t stream) {
    dustin_status st = cand_check(s_draft, draft_units, s_target, target_units, U, unit_ids, C, m_cand, seq_lens, B,
                                  N_max, abar, k, m, n_sink, n_window, "candidate_arr");
    if (st != DUSTIN_OK) return st;
    CHECK(arr != nullptr, DUSTIN_ERR_INVALID_ARG, "candidate_arr: arr is required");
    const bool has_units = draft_units || target_units;
    const bool mat = has_units && (unit_ids != nullptr || (draft_units ? s_draft : s_target) != nullptr);
    const size_t need = cand_layout(C, B, N_max, k, mat).bytes;
    CHECK(ws != nullptr && ws_bytes >= need, DUSTIN_ERR_INVALID_ARG,
          "candidate_arr: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    return cand_run({s_draft, draft_units}, {s_target, target_units}, U, unit_ids, C, m_cand, seq_lens, B, N_max, abar,
                    k, m, n_sink, n_window, arr, arr_mean, (char *)ws, (hipStream_t)stream);
}

size_t dustin_greedy_select_workspace_bytes(int32_t C, int32_t B, int32_t N_max, int32_t k) {
    if (C < 1 || B < 1 || N_max < 1 || k < 1) return 0;
    return align_up(cand_layout(C, B, N_max, k, true).bytes, 256) + align_up((size_t)C * B * sizeof(float), 256) +
           align_up((size_t)C * sizeof(float), 256);
}

dustin_status dustin_greedy_select(const float *units, int32_t U, const int32_t *unit_ids, int32_t C, int32_t side,
                                   const float *s_target_fixed, const int32_t *seq_lens, int32_t B, int32_t N_max,
                                   const float *abar, int32_t k, int32_t m, int32_t n_sink, int32_t n_window,
                                   int32_t max_units, int32_t *chosen, float *curve, int32_t *n_chosen,
                                   float *sum_out, void *ws, size_t ws_bytes, dustin_stream_t stream) {
    CHECK(side == 0 || side == 1, DUSTIN_ERR_INVALID_ARG, "greedy_select: side must be 0 (target) or 1 (draft)");
    CHECK(units != nullptr, DUSTIN_ERR_INVALID_ARG, "greedy_select: units are required");
    CHECK(side == 0 ? s_target_fixed == nullptr : s_target_fixed != nullptr, DUSTIN_ERR_INVALID_ARG,
          "greedy_select: s_target_fixed is required for the draft side and not taken for the target side");
    CHECK(max_units >= 0 && chosen && curve && n_chosen && sum_out, DUSTIN_ERR_INVALID_ARG,
          "greedy_select: max_units >= 0 and the chosen / curve / n_chosen / sum_out outputs are required");
    dustin_status st = cand_check(nullptr, side ? units : nullptr, s_target_fixed, side ? nullptr : units, U, unit_ids,
                                  C, nullptr, seq_lens, B, N_max, abar, k, side ? m : 0, n_sink, n_window,
                                  "greedy_select");
    if (st != DUSTIN_OK) return st;
    const size_t cbytes = align_up(cand_layout(C, B, N_max, k, true).bytes, 256);
    const size_t need = dustin_greedy_select_workspace_bytes(C, B, N_max, k);
    CHECK(ws != nullptr && ws_bytes >= need, DUSTIN_ERR_INVALID_ARG,
          "greedy_select: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    hipStream_t s = (hipStream_t)stream;
    char *wsb = (char *)ws;
    float *arr = (float *)(wsb + cbytes);
    float *mean = (float *)(wsb + cbytes + align_up((size_t)C * B * sizeof(float), 256));
    std::vector<int32_t> ids(C);
    for (int c = 0; c < C; ++c) ids[c] = unit_ids ? unit_ids[c] : c;
    std::vector<float> host(C);
    std::vector<char> used(C, 0);
    auto fetch = [&](int n) -> hipError_t {
        hipError_t e = hipMemcpyAsync(host.data(), mean, (size_t)n * sizeof(float), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        return e;
    };
    const int64_t nel = (int64_t)B * N_max;
    hipError_t e = launch_accumulate(sum_out, nullptr, nel, true, s);   // the empty choice sums to 0
    if (e != hipSuccess) return hip_status(e, "greedy_select clear");
    float best = -__builtin_huge_valf();
    if (side == 1) {
        // the target-history set alone is the objective to beat
        st = cand_run({nullptr, nullptr}, {s_target_fixed, nullptr}, U, nullptr, 1, nullptr, seq_lens, B, N_max, abar,
                      k, 0, n_sink, n_window, arr, mean, wsb, s);
        if (st != DUSTIN_OK) return st;
        if ((e = fetch(1)) != hipSuccess) return hip_status(e, "greedy_select start");
        best = host[0];
    }
    int got = 0;
    for (int it = 0; it < max_units; ++it) {
        const float *base = got ? sum_out : nullptr;
        if (side == 0)
            st = cand_run({nullptr, nullptr}, {base, units}, U, ids.data(), C, nullptr, seq_lens, B, N_max, abar, k, 0,
                          n_sink, n_window, arr, mean, wsb, s);
        else
            st = cand_run({base, units}, {s_target_fixed, nullptr}, U, ids.data(), C, nullptr, seq_lens, B, N_max, abar,
                          k, m, n_sink, n_window, arr, mean, wsb, s);
        if (st != DUSTIN_OK) return st;
        if ((e = fetch(C)) != hipSuccess) return hip_status(e, "greedy_select fetch");
        int top = -1;
        float tv = -__builtin_huge_valf();
        for (int c = 0; c < C; ++c)
            if (!used[c] && host[c] > tv) {
                tv = host[c];
                top = c;
            }
        if (top < 0 || !(tv > best)) break;
        used[top] = 1;
        chosen[got] = top;
        curve[got] = tv;
        best = tv;
        e = launch_accumulate(sum_out, units + (size_t)ids[top] * nel, nel, false, s);
        if (e != hipSuccess) return hip_status(e, "greedy_select accumulate");
        ++got;
    }
    *n_chosen = got;
    return hip_status(hipStreamSynchronize(s), "greedy_select");
}

}  // extern "C"


// ------------------------------------------- measurement kernels
extern "C" {

dustin_status dustin_probe_stream_read(const void *buf, size_t bytes, int32_t nontemporal, uint32_t *sink,
                                       dustin_stream_t stream) {
    CHECK(buf != nullptr && sink != nullptr, DUSTIN_ERR_INVALID_ARG, "probe_stream_read: buf and sink are required");
    CHECK(bytes >= 16 && bytes % 16 == 0, DUSTIN_ERR_INVALID_ARG,
          "probe_stream_read: bytes must be a positive multiple of 16 (got %zu)", bytes);
    return hip_status(launch_probe_stream_read(buf, bytes, nontemporal != 0, sink, 2048, (hipStream_t)stream),
                      "probe_stream_read launch");
}

dustin_status dustin_probe_gather_rows(const void *base, const void *base2, int64_t row_stride, int64_t buf_rows,
                                       const int32_t *rows, int64_t n_rows, int32_t row_bytes,
                                       dustin_stream_t stream) {
    CHECK(base != nullptr && rows != nullptr, DUSTIN_ERR_INVALID_ARG, "probe_gather_rows: base and rows are required");
    CHECK(row_bytes == 64 || row_bytes == 128 || row_bytes == 256 || row_bytes == 512, DUSTIN_ERR_INVALID_ARG,
          "probe_gather_rows: row_bytes %d not one of 64, 128, 256, 512", row_bytes);
    CHECK(row_stride >= row_bytes && row_stride % 16 == 0, DUSTIN_ERR_INVALID_ARG,
          "probe_gather_rows: row_stride %lld must be >= row_bytes and a multiple of 16", (long long)row_stride);
    CHECK(buf_rows >= 1, DUSTIN_ERR_INVALID_ARG, "probe_gather_rows: buf_rows must be >= 1");
    CHECK(n_rows >= 1 && n_rows <= 256LL * 4096, DUSTIN_ERR_INVALID_ARG,
          "probe_gather_rows: n_rows %lld outside 1 .. %lld", (long long)n_rows, 256LL * 4096);
    return hip_status(launch_probe_gather_rows(base, base2, row_stride, buf_rows, rows, n_rows, row_bytes, 256,
                                               (hipStream_t)stream),
                      "probe_gather_rows launch");
}

}  // extern "C"

// ------------------------------------------- allocation-free attention
// dustin_sparse_verify_attn_noalloc keeps what the workspace holds for the
// other entry points (the 64 KiB of arrival counters and the split partials)
// in one static device array per GPU.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per
// device, and is kept per device.
namespace {

constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[DUSTIN_ATTN_SCRATCH_BYTES];

std::mutex g_scratch_mu;
char *g_scratch_ptr[kScratchDevices];

__global__ __launch_bounds__(256) void scratch_zero_counters(int32_t *c, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) c[i] = 0;
}

// The scratch's device address on the current device.  The first call on a
// device looks it up and zero-fills the counter region with a kernel on
// `s` (every attention launch leaves the counters at zero again, so this is
// the only clear that is needed).
dustin_status scratch_on_current_device(hipStream_t s, char **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "sparse_verify_attn_noalloc: hipGetDevice");
    CHECK(dev >= 0 && dev < kScratchDevices, DUSTIN_ERR_UNSUPPORTED,
          "sparse_verify_attn_noalloc: device %d outside the %d the scratch table holds", dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "sparse_verify_attn_noalloc: hipGetSymbolAddress(scratch)");
        hipLaunchKernelGGL(scratch_zero_counters, dim3(kAttnCounterSlots / 256), dim3(256), 0, s, (int32_t *)ptr,
                           kAttnCounterSlots);
        if ((e = hipGetLastError()) != hipSuccess)
            return hip_status(e, "sparse_verify_attn_noalloc: clearing the scratch counters");
        g_scratch_ptr[dev] = (char *)ptr;
    }
    *out = g_scratch_ptr[dev];
    return DUSTIN_OK;
}

}  // namespace

extern "C" {

dustin_status dustin_sparse_verify_attn_noalloc(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                                                const int32_t *idx, const int32_t *count, int32_t k, float scale,
                                                void *out, float *lse, dustin_stream_t stream) {
    static const char *name = "sparse_verify_attn_noalloc";
    AttnArgs a;
    AttnPlan p;
    dustin_status st =
        attn_prepare(name, q, w, H_q, kv, idx, count, k, scale, out, lse, nullptr, 0, 0, a, p, true);
    if (st != DUSTIN_OK) return st;
    CHECK(p.ws_bytes <= (size_t)DUSTIN_ATTN_SCRATCH_BYTES, DUSTIN_ERR_UNSUPPORTED,
          "%s: this shape needs %zu bytes of scratch, the static scratch holds %zu "
          "(dustin_sparse_verify_attn takes a workspace of any size)",
          name, p.ws_bytes, (size_t)DUSTIN_ATTN_SCRATCH_BYTES);
    char *base = nullptr;
    if ((st = scratch_on_current_device((hipStream_t)stream, &base)) != DUSTIN_OK) return st;
    bind_attn_workspace(a, p, base);
    return hip_status(launch_attn(a, p, (hipStream_t)stream), "sparse_verify_attn_noalloc launch");
}

}  // extern "C"
