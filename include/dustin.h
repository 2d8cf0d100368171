/*
 * dustin.h -- C ABI of the MI355X (gfx950) sparse-verification step.
 *
 * The step is the target-side verification of long-context, multi-batch
 * speculative decoding described for "Dustin: Draft-Augmented Sparse
 * Verification for Efficient Long-Context Generation with Speculative
 * Decoding" (arXiv 2606.24957):
 *   1. hybrid token-importance scoring   -> dustin_score
 *   2. one global TopK index set per sequence, shared by every layer and
 *      head (protected sink/window tokens, draft top-m, target fill)
 *                                        -> dustin_topk
 *   3. grouped-query attention of the w window tokens over the selected
 *      K/V rows only                     -> dustin_sparse_verify_attn
 *      (history only) or dustin_verify_attn (history set plus the window's
 *      own rows, causally), with dustin_append_window_kv writing the window
 *      into the cache first (dustin_verify_attn_append: both in one call)
 *      and dustin_commit_window keeping the accepted tokens afterwards
 *   plus the evaluator of the translation's section 3.1 (attention recovery
 *   rate):                               -> dustin_window_attn, dustin_arr,
 *   and the policy comparison of its sections 3.2-3.3
 *                                        -> dustin_window_mean, dustin_policy_sweep
 *   and the page-level estimator the pages compare scoring costs with
 *                                        -> dustin_page_bounds, dustin_page_scores
 *   and the offline configuration search of blog section 2.4
 *                                        -> dustin_head_scores, dustin_candidate_arr,
 *                                           dustin_greedy_select
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers unless marked "host"; all tensors are
 *   dense row-major with the shapes given.  The caller owns every buffer,
 *   including the workspace; the library never allocates or frees memory.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *   default stream).  Nothing synchronises; device-side faults surface at
 *   the caller's next synchronisation.
 * - All argument checks run on the host before any HIP call, so every
 *   DUSTIN_ERR_INVALID_ARG / DUSTIN_ERR_UNSUPPORTED path works without a GPU.
 *   Values that live in device memory (sequence lengths, page tables, index
 *   lists) cannot be checked on the host; kernels clamp them: lengths to
 *   [0, N_max], index entries outside [0, n_b) and page ids outside
 *   [0, num_pages) are treated as absent (never dereferenced).
 * - Workspace: pass at least the byte count the matching *_workspace_bytes()
 *   function returns for the same shape.  dustin_sparse_verify_attn,
 *   dustin_verify_attn, dustin_verify_attn_append, dustin_window_attn and
 *   dustin_policy_sweep keep
 *   arrival counters in the first 64 KiB of their workspace (one slot per
 *   (sequence, KV head), so B * H_kv <= 16384): that region must be
 *   zero-filled before its first
 *   use and every call leaves it zero again, so one workspace may serve
 *   successive calls of these entry points of any shapes, but it must
 *   not be handed to another entry point in between.  The other entry
 *   points make no assumption about workspace contents.
 *   Calls that may overlap in time must not share a workspace.
 * - Outputs are bitwise deterministic for fixed inputs and shapes.
 * - Functions are stateless and reentrant; dustin_last_error() is
 *   thread-local.
 */
#ifndef DUSTIN_H
#define DUSTIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DUSTIN_ABI_VERSION 7

typedef enum dustin_status {
    DUSTIN_OK = 0,
    DUSTIN_ERR_INVALID_ARG = 1, /* bad shape, null required pointer, small workspace */
    DUSTIN_ERR_UNSUPPORTED = 2, /* valid request the library does not implement */
    DUSTIN_ERR_HIP = 3          /* a HIP runtime call failed; see dustin_last_error() */
} dustin_status;

typedef enum dustin_dtype {
    DUSTIN_F32 = 0,  /* float32 storage, float32 arithmetic */
    DUSTIN_BF16 = 1  /* bfloat16 storage, float32 accumulation */
} dustin_dtype;

/* hipStream_t without pulling in the HIP headers. */
typedef struct ihipStream_t *dustin_stream_t;

/*
 * One layer's KV cache (the blog's Fig. 5: the full target or draft cache
 * stays resident; a verification step only reads part of it).
 *
 *  page_size == 0 (contiguous):  k, v are [B][N_max][H_kv][head_dim]
 *  page_size == 16 (paged):      k, v are [num_pages][16][H_kv][head_dim];
 *      logical position j of sequence b lives in physical page
 *      page_table[b * max_pages + j / 16], slot j % 16.
 *  seq_lens [B] (device, int32): n_b = |V_i|, the valid history length of
 *      sequence b; rows at positions >= n_b are never read.
 *  v may be NULL where only keys are needed (scoring, dustin_window_attn).
 *  head_dim must be 32, 64 or 128.
 */
typedef struct dustin_kv {
    const void *k;
    const void *v;
    int32_t dtype;              /* dustin_dtype */
    int32_t B;
    int32_t H_kv;
    int32_t head_dim;
    int32_t N_max;
    const int32_t *seq_lens;    /* device [B] */
    int32_t page_size;          /* 0 or 16 */
    const int32_t *page_table;  /* device [B][max_pages]; NULL when contiguous */
    int32_t max_pages;
    int32_t num_pages;          /* pages in the pool (bounds page ids) */
} dustin_kv;

/*
 * dustin_score -- hybrid token-importance vectors (blog section 2.2; the
 * scored target heads are the searched subset of section 2.4).
 *
 *   S_Draft[b][j]  = sum over draft layers l < L_d, draft heads h < H_d and
 *                    draft steps g < gamma of
 *                    softmax_{j < n_b}(scale_draft * q_draft[b][l][g][h] . Kd_l[b][j][h / G_d])
 *                    with G_d = H_d / draft_layers[l].H_kv;
 *   S_Target[b][j] = sum over r < S of
 *                    softmax_{j < n_b}(scale_target * q_hist[b][r] . Kt_{L(r)}[b][j][H(r) / G])
 *                    where (L(r), H(r)) = (sub_heads[2r], sub_heads[2r+1]) and
 *                    G = H_t / target_layers[L(r)].H_kv.
 * The softmax runs over the history positions only.  q_hist holds the
 * target's most recent query (history distance 1, translation section 3.2).
 *
 *  draft_layers   host [L_d] descriptors (k used; same B, N_max, H_kv,
 *                 head_dim, dtype, paging for all layers); B <= 1024
 *  q_draft        [B][L_d][gamma][H_d][d_draft], draft dtype
 *  target_layers  host [L_t] descriptors (k used; same B, N_max as draft)
 *  q_hist         [B][S][d_target], target dtype
 *  sub_heads      host [S][2] (layer, head) pairs, 0 <= layer < L_t,
 *                 0 <= head < H_t
 *  scale_*        softmax scale; 0 means 1/sqrt(head_dim)
 *  draft_lse      nullable, device [B][L_d][gamma][H_d] float32: the row
 *                 normalisers ln sum_{j < n_b} exp(scale_draft * q . k_j) of
 *                 the draft softmaxes above (what the draft model's own
 *                 attention over the history computes for these queries;
 *                 dustin_draft_row_lse gives the same values).  When given,
 *                 S_Draft reads the draft keys once, using these normalisers
 *                 as they are, instead of twice; -inf (or any non-finite
 *                 value) marks an empty row
 *  s_draft        [B][N_max] float32 out, 0 at j >= n_b; NULL or L_d == 0
 *                 skips the draft side
 *  s_target       [B][N_max] float32 out; NULL or S == 0 skips it
 * Sequence lengths come from the first descriptor used (draft layer 0, else
 * target layer 0); every descriptor must describe the same sequences.
 */
dustin_status dustin_score(const dustin_kv *draft_layers, int32_t L_d,
                           const void *q_draft, int32_t H_d, int32_t gamma,
                           const dustin_kv *target_layers, int32_t L_t,
                           const void *q_hist, const int32_t *sub_heads,
                           int32_t S, int32_t H_t,
                           float scale_draft, float scale_target,
                           const float *draft_lse,
                           float *s_draft, float *s_target,
                           void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_score_workspace_bytes(int32_t B, int32_t N_max, int32_t L_d,
                                    int32_t H_d, int32_t gamma, int32_t S);

/*
 * dustin_draft_row_lse -- the row normalisers of S_Draft's softmaxes (blog
 * section 2.2): lse_out[b][l][g][h] = ln sum_{j < n_b} exp(scale_draft *
 * q_draft[b][l][g][h] . Kd_l[b][j][h / G_d]), -inf for an empty history.
 * Arguments and workspace as for dustin_score's draft side (workspace size
 * dustin_score_workspace_bytes(B, N_max, L_d, H_d, gamma, 0)); lse_out is
 * device [B][L_d][gamma][H_d] float32.  One read of the draft keys.
 */
dustin_status dustin_draft_row_lse(const dustin_kv *draft_layers, int32_t L_d,
                                   const void *q_draft, int32_t H_d, int32_t gamma,
                                   float scale_draft, float *lse_out,
                                   void *ws, size_t ws_bytes, dustin_stream_t stream);

/*
 * dustin_topk -- the per-sequence verification set I_verify (blog section
 * 2.3), global across layers and heads (blog section 2.2):
 *   P = [0, min(n_sink, n)) U [max(0, n - n_window), n)      protected
 *   D = the m' positions outside P with the largest S_Draft   draft tier
 *   T = the positions outside P u D with the largest S_Target filling the
 *       budget                                                 target tier
 * with m' = min(m, k - |P|, n - |P|), |I| = min(k, n); ties go to the lower
 * position.  s_draft == NULL means m' = 0; s_target == NULL means the draft
 * tier fills the budget.  The SD oracle of the translation's Eq. (3) is this
 * call on the window-mean attention with m = n_sink = n_window = 0.
 *
 *  s_draft, s_target  [B][N_max] float32, non-negative (positions >= n_b
 *                     are ignored)
 *  seq_lens           [B] device int32
 *  idx   out [B][k] int32: selected positions in ascending order, -1 padded
 *  count out [B] int32 = min(k, n_b)
 *  tier  out, nullable [B][k] int8: 0 protected, 1 draft, 2 target, -1 pad
 * Requires 1 <= k, 0 <= m, n_sink, n_window >= 0, n_sink + n_window <= k.
 */
dustin_status dustin_topk(const float *s_draft, const float *s_target,
                          const int32_t *seq_lens, int32_t B, int32_t N_max,
                          int32_t k, int32_t m, int32_t n_sink, int32_t n_window,
                          int32_t *idx, int32_t *count, int8_t *tier,
                          void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_topk_workspace_bytes(int32_t B, int32_t N_max, int32_t k);

/*
 * dustin_sparse_verify_attn -- Stage 2 of the blog's Fig. 5: attention of
 * the w window queries over the compressed KV (only the selected rows).
 *   O[b][s][h] = sum_{j in I_b} softmax_{j in I_b}(scale * q[b][s][h] . K[b][j][h/G]) V[b][j][h/G]
 *   lse[b][s][h] = ln sum_{j in I_b} exp(scale * q[b][s][h] . K[b][j][h/G])
 * with G = H_q / kv->H_kv and I_b = idx[b][0 .. count[b]).
 * idx == NULL gives dense full-cache attention over j < n_b (the blog's
 * "Full Cache" baseline of Fig. 7); count is then ignored and k must be 0.
 *
 *  q     [B][w][H_q][head_dim], kv dtype
 *  kv    k and v required
 *  idx   [B][k] int32 positions (any order, no duplicates), or NULL
 *  count [B] int32 (entries beyond count[b] are ignored)
 *  scale 0 means 1/sqrt(head_dim)
 *  out   [B][w][H_q][head_dim], kv dtype; an empty set gives 0
 *  lse   nullable [B][w][H_q] float32; an empty set gives -inf
 * Requires w * (H_q / H_kv) <= 64.  head_dim 32, 64 or 128 in either dtype
 * (bfloat16 head_dim 32 pads up to 32 query rows per KV head); the same
 * holds for every attention entry point below.
 */
dustin_status dustin_sparse_verify_attn(const void *q, int32_t w, int32_t H_q,
                                        const dustin_kv *kv, const int32_t *idx,
                                        const int32_t *count, int32_t k, float scale,
                                        void *out, float *lse,
                                        void *ws, size_t ws_bytes, dustin_stream_t stream);

/* k_or_n: the k passed to the call, or N_max for the dense (idx == NULL) form. */
size_t dustin_attn_workspace_bytes(int32_t B, int32_t w, int32_t H_q, int32_t H_kv,
                                   int32_t head_dim, int32_t k_or_n);

/*
 * dustin_sparse_verify_attn_noalloc -- dustin_sparse_verify_attn for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments,
 * results and errors, minus the workspace.  The call allocates nothing.
 * Its arrival counters and split partials live in a static device array of
 * DUSTIN_ATTN_SCRATCH_BYTES per GPU (the library's, held from the first
 * call on that GPU until the process ends), on the current device; `stream`
 * must belong to it.  A shape whose workspace
 * (dustin_attn_workspace_bytes) exceeds that size is refused with
 * DUSTIN_ERR_UNSUPPORTED before any HIP call.  The first call on a device
 * also enqueues one small kernel on `stream` that zero-fills the counters;
 * every call leaves them at zero.  All calls on one GPU share the array:
 * calls that may overlap in time on one GPU (other streams, other threads)
 * race and must be serialised by the caller.
 */
#define DUSTIN_ATTN_SCRATCH_BYTES (32u << 20)
dustin_status dustin_sparse_verify_attn_noalloc(const void *q, int32_t w, int32_t H_q,
                                                const dustin_kv *kv, const int32_t *idx,
                                                const int32_t *count, int32_t k, float scale,
                                                void *out, float *lse, dustin_stream_t stream);

/*
 * dustin_append_window_kv -- writes the w draft tokens' keys and values into
 * the target cache right after each history, as Stage 2 of the blog's Fig. 5
 * does before verifying them: row n_b + t of sequence b receives
 * k_win[b][t] / v_win[b][t] for t < w.  seq_lens is read, not changed.
 *
 *  kv     k and v required; rows at positions >= N_max are not written
 *         (the caller keeps N_max >= n_b + w), and in a paged cache a
 *         position whose page id is outside [0, num_pages) is skipped
 *  k_win  [B][w][H_kv][head_dim], kv dtype
 *  v_win  [B][w][H_kv][head_dim], kv dtype
 * kv->k, kv->v, k_win and v_win must be 16-byte aligned.
 */
dustin_status dustin_append_window_kv(const dustin_kv *kv, const void *k_win, const void *v_win,
                                      int32_t w, dustin_stream_t stream);

/*
 * dustin_verify_attn -- the whole attention of one verification step (blog,
 * Fig. 5, Stage 2): window query s of sequence b attends the selected
 * history rows I_b and the window's own rows n_b .. n_b + s (already in the
 * cache through dustin_append_window_kv), i.e. a causal block over the
 * window:
 *   J_{b,s} = I_b  U  { n_b + t : 0 <= t <= s }
 *   O[b][s][h]   = sum_{j in J_{b,s}} softmax_j(scale * q[b][s][h] . K[b][j][h/G]) V[b][j][h/G]
 *   lse[b][s][h] = ln sum_{j in J_{b,s}} exp(scale * q[b][s][h] . K[b][j][h/G])
 * Arguments, layouts and errors as for dustin_sparse_verify_attn; idx ==
 * NULL gives the dense form I_b = { j < n_b } (the "Full Cache" step).
 * Index entries at or past n_b are ignored (the window rows are added by
 * the call itself), and window rows at positions >= N_max are left out.
 * Workspace: dustin_verify_attn_workspace_bytes for the same shape.
 */
dustin_status dustin_verify_attn(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                                 const int32_t *idx, const int32_t *count, int32_t k, float scale,
                                 void *out, float *lse, void *ws, size_t ws_bytes,
                                 dustin_stream_t stream);

/*
 * dustin_verify_attn_append -- dustin_append_window_kv followed by
 * dustin_verify_attn, in one launch for bfloat16 caches (two for float32):
 * the same cache contents and bitwise the same out / lse as the two calls
 * in order.  The window's own rows are read from k_win / v_win, and the
 * first token split of each (sequence, KV head) also writes them into the
 * cache rows n_b .. n_b + w - 1 (rows at positions >= N_max, or whose page
 * id is outside [0, num_pages), are neither written nor attended, as in the
 * separate calls).  Arguments as for dustin_verify_attn, plus k_win /
 * v_win as for dustin_append_window_kv; same workspace
 * (dustin_verify_attn_workspace_bytes).  kv->k, kv->v, k_win and v_win must
 * be 16-byte aligned.
 */
dustin_status dustin_verify_attn_append(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                                        const void *k_win, const void *v_win, const int32_t *idx,
                                        const int32_t *count, int32_t k, float scale, void *out, float *lse,
                                        void *ws, size_t ws_bytes, dustin_stream_t stream);

/* k_or_n: the k passed to the call, or N_max for the dense (idx == NULL) form. */
size_t dustin_verify_attn_workspace_bytes(int32_t B, int32_t w, int32_t H_q, int32_t H_kv,
                                          int32_t head_dim, int32_t k_or_n);

/*
 * dustin_commit_window -- the end of a verification step (blog, Fig. 5,
 * Stage 2): the accepted tokens' rows stay in the cache and the rejected
 * ones are dropped, so seq_lens[b] += clamp(accepted[b], 0, w).  The rows of
 * rejected tokens then lie past the new length and are overwritten by the
 * next dustin_append_window_kv.
 *
 *  seq_lens  [B] int32, updated in place
 *  accepted  [B] int32 accepted-token counts
 */
dustin_status dustin_commit_window(int32_t *seq_lens, const int32_t *accepted, int32_t B,
                                   int32_t w, dustin_stream_t stream);

/*
 * dustin_window_attn -- the full-cache attention weights A_{i+s,j} of the
 * translation's section 3.1 for every window step s < w, as the mean over
 * the H_q query heads of one layer of each head's softmax over the history
 * j < n_b (so sum_j A[b][s][j] = 1).
 *
 *  q   [B][w][H_q][head_dim], kv dtype
 *  A   out [B][w][N_max] float32, 0 at j >= n_b
 *
 * w <= 16.  bfloat16 caches (B <= 1024): G = H_q / H_kv <= 64; the window is
 * processed in slices of min(4, 64 / G) steps, two reads of K per slice.
 * float32 caches: w * G <= 64 (the attention kernel's limit).  Anything else
 * returns DUSTIN_ERR_UNSUPPORTED.
 */
dustin_status dustin_window_attn(const void *q, int32_t w, int32_t H_q,
                                 const dustin_kv *kv, float scale, float *A,
                                 void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_window_attn_workspace_bytes(int32_t B, int32_t w, int32_t H_q,
                                          int32_t H_kv, int32_t head_dim, int32_t N_max);

/*
 * dustin_arr -- attention recovery rate of an index set (translation section
 * 3.1): Eq. (1) arr_step[b][s] = sum_{j in I_b} A[b][s][j] and Eq. (2)
 * arr_window[b] = (1/w) sum_s arr_step[b][s].  Entries of idx beyond
 * count[b], negative or >= n_b are ignored; duplicates count once per entry.
 *
 *  A          [B][w][N_max] float32 (e.g. from dustin_window_attn)
 *  idx, count as produced by dustin_topk
 *  arr_step   out [B][w] float32 (nullable)
 *  arr_window out [B] float32 (nullable)
 */
dustin_status dustin_arr(const float *A, const int32_t *seq_lens, int32_t B, int32_t w,
                         int32_t N_max, const int32_t *idx, const int32_t *count, int32_t k,
                         float *arr_step, float *arr_window, dustin_stream_t stream);

/*
 * dustin_window_mean -- the averaged future attention of Eq. (3) in the
 * translation's section 3.1: Abar[b][j] = (1/w) sum_{s < w} A[b][s][j]
 * (TopK_k of Abar is the SD oracle's set, Eq. (4)).
 *
 *  A     [B][w][N_max] float32 (e.g. from dustin_window_attn)
 *  Abar  out [B][N_max] float32
 */
dustin_status dustin_window_mean(const float *A, int32_t B, int32_t w, int32_t N_max, float *Abar,
                                 dustin_stream_t stream);

/*
 * dustin_policy_sweep -- windowed ARR (Eq. 2) of the selection policies the
 * pages compare, at every budget ks[i] (translation sections 3.2-3.3,
 * Figs. 2-3, and the variants of the blog's Table 3), per sequence.  The
 * ground truth is A of the w window queries (Eq. 1, head mean over one
 * target layer).  Output rows:
 *   row 0                   SD oracle: TopK_k of Abar (Eq. 3-4)
 *   rows 1 .. n_past        history: TopK_k of A_{i-delta,.}, the head-mean
 *                           full-cache attention of past query p (Fig. 2)
 *   row n_past + 1          draft lookahead alone: TopK_k of S_Draft (Fig. 3)
 *   rows n_past + 2 .. + 4  the dustin_topk verification set with m = 0
 *                           (Dustin-T), m = k - n_sink - n_window (Dustin-D)
 *                           and m = m_hybrid[i] (Dustin-H)
 * Ties in every TopK: higher score first, then lower position.
 *
 *  q_window  [B][w][H_q][head_dim], kv dtype (w <= 16)
 *  q_past    [n_past][B][H_q][head_dim], kv dtype; NULL when n_past == 0
 *            (n_past <= 64)
 *  kv        one target layer (k used)
 *  s_draft, s_target  [B][N_max] float32 (e.g. from dustin_score)
 *  ks, m_hybrid  host [nk]; every k >= n_sink + n_window, 0 <= m_hybrid <= k
 *  arr       out [n_past + 5][nk][B] float32
 *  ws        dustin_policy_sweep_workspace_bytes(..., max k) bytes; its first
 *            64 KiB are arrival counters under the same rules as the
 *            attention workspaces (zero-filled before first use, left zero)
 * The calls run in order on `stream`.
 */
dustin_status dustin_policy_sweep(const void *q_window, int32_t w, const void *q_past, int32_t n_past,
                                  int32_t H_q, const dustin_kv *kv, const float *s_draft,
                                  const float *s_target, const int32_t *ks, const int32_t *m_hybrid,
                                  int32_t nk, int32_t n_sink, int32_t n_window, float scale, float *arr,
                                  void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_policy_sweep_workspace_bytes(int32_t B, int32_t w, int32_t n_past, int32_t H_q,
                                           int32_t H_kv, int32_t head_dim, int32_t N_max, int32_t k_max);

/*
 * dustin_page_bounds -- page statistics of the page-level estimator the
 * pages compare Dustin's scoring with (Quest in the translation's related
 * work: pages scored from cheap min/max key statistics; Quest-16 in the
 * blog's Fig. 8): for every 16-position page p and KV head g,
 *   kmin[b][p][g][d] = min_{j in page p, j < n_b} K[b][j][g][d], kmax likewise.
 * Pages with no position below n_b are written as 0.
 *
 *  kv          k used (contiguous, or paged with its own 16-position pages)
 *  kmin, kmax  out [B][ceil(N_max / 16)][H_kv][head_dim], kv dtype (exact:
 *              the bounds are stored values); 16-byte aligned
 */
dustin_status dustin_page_bounds(const dustin_kv *kv, void *kmin, void *kmax, dustin_stream_t stream);

/*
 * dustin_page_scores -- page criticality from the bounds alone (no QK^T):
 *   scores[b][p] = scale * sum_{s < w} sum_{h < H_q} sum_d
 *                  max(q[b][s][h][d] * kmin[b][p][g(h)][d], q[b][s][h][d] * kmax[b][p][g(h)][d])
 * (the per-head bound of scale * q . k over the page's box, summed over the
 * window steps and heads for one global page set); 0 for pages with no
 * position below n_b.
 *
 *  q       [B][w][H_q][head_dim], kv dtype; 16-byte aligned
 *  kmin, kmax  from dustin_page_bounds
 *  scale   0 means 1/sqrt(head_dim)
 *  scores  out [B][ceil(N_max / 16)] float32
 *  ws      device scratch, >= dustin_page_scores_workspace_bytes(B, H_kv,
 *          head_dim), 16-byte aligned; its contents need no initialisation
 *
 * Both calls need H_kv * head_dim <= 4096 (else DUSTIN_ERR_UNSUPPORTED).
 */
dustin_status dustin_page_scores(const void *q, int32_t w, int32_t H_q, const dustin_kv *kv,
                                 const void *kmin, const void *kmax, float scale, float *scores,
                                 void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_page_scores_workspace_bytes(int32_t B, int32_t H_kv, int32_t head_dim);

/*
 * Offline configuration search (blog section 2.4 and Fig. 6: a (layer, head)
 * score matrix with its head TopK, greedy target layers/heads, greedy draft
 * layers with the target fixed, then the draft/target split m; the
 * objective is the windowed ARR of translation section 3.1, Eq. 2).  These
 * calls run on profiling data, not on the verification step.
 *
 * Objective of a verification set I of sequence b: Eq. 2 is linear in A, so
 *   (1/w) sum_s sum_{j in I} A[s][j] = sum_{j in I} abar[b][j]
 * with abar the window-step mean of A (dustin_window_mean), averaged over the
 * target layers the set has to serve.  A configuration's objective is the
 * mean over the profiling batch.
 */

/*
 * dustin_head_scores -- per-head S_Target rows: the softmax over the history
 * of every listed (layer, head) pair's query, not summed,
 *   out[r][b][j] = softmax_{j < n_b}(scale * q_hist[b][r] . Kt_{L(r)}[b][j][H(r) / G]),
 * 0 at j >= n_b.  Arguments as for dustin_score's target side (up to 64 rows
 * over up to 8 distinct layers per call); out [S][B][N_max] float32.
 */
dustin_status dustin_head_scores(const dustin_kv *target_layers, int32_t L_t, const void *q_hist,
                                 const int32_t *sub_heads, int32_t S, int32_t H_t, float scale, float *out,
                                 void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_head_scores_workspace_bytes(int32_t B, int32_t N_max, int32_t S);

/*
 * dustin_candidate_arr -- objective of C candidate configurations.  For
 * candidate c and sequence b the verification set is dustin_topk's (blog
 * section 2.3) on
 *   S_Draft  = s_draft[b]  + draft_units[u(c)][b]    (side absent if both NULL)
 *   S_Target = s_target[b] + target_units[u(c)][b]
 * with m = m_cand[c] (host, nullable; else m), u(c) = unit_ids[c] (host,
 * nullable; else c), and
 *   arr[c][b] = sum_{j in I} abar[b][j],   arr_mean[c] = mean_b arr[c][b].
 *
 *  s_draft, s_target       [B][N_max] float32 base vectors, nullable
 *  draft_units / target_units  [U][B][N_max] float32, at most one side
 *  seq_lens                [B] device int32
 *  abar                    [B][N_max] float32
 *  arr                     out [C][B] float32; arr_mean out [C] or NULL
 *  ws                      >= dustin_candidate_arr_workspace_bytes(C, B,
 *                          N_max, k, materialize), materialize = 1 when a
 *                          side has units and (a base or unit_ids)
 * Ties follow dustin_topk.  C * B <= 2^24.
 */
dustin_status dustin_candidate_arr(const float *s_draft, const float *draft_units, const float *s_target,
                                   const float *target_units, int32_t U, const int32_t *unit_ids, int32_t C,
                                   const int32_t *m_cand, const int32_t *seq_lens, int32_t B, int32_t N_max,
                                   const float *abar, int32_t k, int32_t m, int32_t n_sink, int32_t n_window,
                                   float *arr, float *arr_mean, void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_candidate_arr_workspace_bytes(int32_t C, int32_t B, int32_t N_max, int32_t k, int32_t materialize);

/*
 * dustin_greedy_select -- greedy forward selection (blog section 2.4, steps
 * 1 and 2) over C candidate units of one side:
 *   side 0 (target): units are S_Target vectors; sets use m = 0 (target
 *     history); the first unit is always taken; s_target_fixed must be NULL.
 *   side 1 (draft): units are S_Draft vectors, S_Target = s_target_fixed,
 *     draft budget m; the empty choice (the target-history set) is the
 *     objective to beat.
 * Each round evaluates every remaining candidate (dustin_candidate_arr with
 * the chosen units' sum as the base) and adds the one with the largest
 * batch-mean objective (ties: lower candidate index); it stops after
 * max_units additions or when no candidate improves the objective strictly.
 *
 *  units        [U][B][N_max] float32; unit_ids host [C] into them (NULL: 0..C-1)
 *  chosen       host out [max_units]: candidate indices (into the C list) in order
 *  curve        host out [max_units]: objective after each addition
 *  n_chosen     host out
 *  sum_out      device out [B][N_max]: sum of the chosen units (0 if none)
 *  ws           >= dustin_greedy_select_workspace_bytes(C, B, N_max, k)
 * Blocking: the call waits for the stream after every round (it reads the
 * objectives back), so it cannot be captured into a graph.
 */
dustin_status dustin_greedy_select(const float *units, int32_t U, const int32_t *unit_ids, int32_t C, int32_t side,
                                   const float *s_target_fixed, const int32_t *seq_lens, int32_t B, int32_t N_max,
                                   const float *abar, int32_t k, int32_t m, int32_t n_sink, int32_t n_window,
                                   int32_t max_units, int32_t *chosen, float *curve, int32_t *n_chosen,
                                   float *sum_out, void *ws, size_t ws_bytes, dustin_stream_t stream);

size_t dustin_greedy_select_workspace_bytes(int32_t C, int32_t B, int32_t N_max, int32_t k);

/*
 * Measurement kernels.  They compute nothing of the method: they give the
 * achievable HBM rates that the step's kernels are compared with, beside
 * the 8 TB/s peak of the part.
 *
 * dustin_probe_stream_read -- reads every 16-byte piece of `buf` once
 * (grid-stride, 2048 work-groups of 256 lanes, four loads in flight per
 * lane), with the nontemporal cache policy of the scoring passes
 * (nontemporal != 0) or the default policy.
 *  buf   device, `bytes` bytes (a positive multiple of 16)
 *  sink  device [2048] uint32; written only in the impossible case that the
 *        folded data equals a marker (it keeps the loads from being dropped)
 *
 * dustin_probe_gather_rows -- gathers rows[0 .. n_rows) (row numbers,
 * clamped to [0, buf_rows)) of `row_bytes` bytes each, at row r of base
 * (byte r * row_stride) and, when base2 is not NULL, at the same row of
 * base2, into LDS with global->LDS DMA: the access pattern of the
 * verification attention's K/V gather (256 work-groups of 8 waves, a
 * four-stage 32 KiB ring each, no arithmetic).  Work-group g takes the
 * rows g * ceil(n_rows / 256) .. in list order.
 *  row_bytes   64, 128, 256 or 512; row_stride >= row_bytes, a multiple of 16
 *  n_rows      1 .. 256 * 4096
 * Both return DUSTIN_ERR_INVALID_ARG for the conditions above, checked on
 * the host before any HIP call.
 */
dustin_status dustin_probe_stream_read(const void *buf, size_t bytes, int32_t nontemporal, uint32_t *sink,
                                       dustin_stream_t stream);
dustin_status dustin_probe_gather_rows(const void *base, const void *base2, int64_t row_stride, int64_t buf_rows,
                                       const int32_t *rows, int64_t n_rows, int32_t row_bytes,
                                       dustin_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char *dustin_status_string(dustin_status status);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char *dustin_last_error(void);

/* DUSTIN_ABI_VERSION of the loaded library. */
int32_t dustin_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DUSTIN_H */
