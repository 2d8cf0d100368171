// Hybrid token-importance scoring (Dustin blog section 2.2; scored target
// heads restricted to a small searched subset, section 2.4) for gfx950.
//
//   S_Target[b][j] = sum_r softmax_j(scale * q_hist[b][r] . K_{L(r)}[b][j][kv(r)])
//   S_Draft[b][j]  = sum_{l,h,g} softmax_j(scale_d * q_draft[b][l][g][h] . Kd_l[b][j][h/G_d])
//
// Each softmax is normalised over the whole history j < n_b before the sum,
// so every row needs its global max and sum.  Both sides therefore work in
// two steps:
//   1. a streaming pass over K that produces, per row and per 256-position
//      chunk, the chunk max and sum of exp2 (log2 domain);
//   2. a second step that turns the chunk statistics into each row's
//      log-sum-exp and accumulates the normalised probabilities per position.
// Target side: step 1 also keeps the (few) logits, so step 2 reads logits
// instead of K.  Draft side: 28 rows per K row make stored logits larger than
// K itself, so step 2 recomputes the logits from K with MFMA.
//
// Work-group -> data mapping: one 256-lane work-group per (sequence, unit,
// 256-position chunk) in step 1; one per (sequence, chunk) in the draft's
// step 2, which loops over all draft (layer, KV head) units and sums in a
// fixed order, so S_Draft is bitwise deterministic without atomics.

#include "common.h"
#include "internal.h"

#include <type_traits>

namespace dustin {

constexpr int CH = kScoreChunk;
constexpr int kScoreGroups = 1024;   // persistent work-groups (four per CU)

__device__ __forceinline__ int sl_len(const KvView &kv, int b) {
    return min(max(kv.seq_lens[b], 0), kv.N_max);
}

// Byte pointer to the head row (b, j, h) of one layer's K, or nullptr when a
// page id is out of range.
__device__ __forceinline__ const char *krow(const KvView &kv, int b, int j, int h, int esz) {
    int64_t r;
    if (kv.page_size == 0) {
        r = (int64_t)b * kv.N_max + j;
    } else {
        const int pg = kv.page_table[(int64_t)b * kv.max_pages + (j >> 4)];
        if (pg < 0 || pg >= kv.num_pages) return nullptr;
        r = (int64_t)pg * 16 + (j & 15);
    }
    return kv.k + ((r * kv.Hkv + h) * kv.D) * esz;
}

// Load the 16-byte slice `slice` of a head row as floats (8 bf16 or 4 f32).
template <bool F32>
__device__ __forceinline__ void load_slice(const char *row, int slice, float (&x)[8]) {
    if (row == nullptr) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
        return;
    }
    const u32x4 v = ld_stream16(row + slice * 16);
    if constexpr (F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
#pragma unroll
        for (int i = 4; i < 8; ++i) x[i] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(v[i] << 16);
            x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
}

// ---------------------------------------------------------------------------
// Generic VALU statistics pass.  A "unit" is one (layer view, KV head) with up
// to 8 query rows sharing it.  Lanes are grouped LPI per position (16 bytes
// per lane); each group computes the dot products of one K row with the
// unit's rows.

struct UnitTable {
    int32_t n_units;
    int32_t view[kMaxScoreRows];     // index into the KvView array
    int32_t kvh[kMaxScoreRows];
    int32_t row0[kMaxScoreRows];     // first global row id of the unit
    int32_t nrow[kMaxScoreRows];     // rows in the unit (<= 8)
};

template <bool F32, int D, int NV>
struct ValuStatsParams {
    KvView kv[NV];
    UnitTable ut;
    const char *q;                   // row r of sequence b at q + (b * q_bstride + qoff[r]) * esz
    int64_t q_bstride;
    int32_t qoff[kMaxScoreQoff];
    int32_t total_rows;
    float scale_log2;
    float *stat;                     // [B][total_rows][nchunk][2]
    float *logit;                    // [B][total_rows][N_max] or nullptr
    int32_t nchunk, N_max;
};

template <bool F32, int D, int NV>
__global__ __launch_bounds__(256) void unit_stats_valu(ValuStatsParams<F32, D, NV> p) {
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int LPI = D * ESZ / 16;         // lanes per position
    constexpr int EPL = 16 / ESZ;             // elements per lane
    constexpr int IPP = 256 / LPI;            // positions per pass
    __shared__ float qs[8][D];
    __shared__ float lg[8][CH];
    __shared__ int pgs[CH / 16];   // paged caches: the chunk's page ids

    const int chunk = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const KvView &kv = p.kv[p.ut.view[u]];
    const int kvh = p.ut.kvh[u], row0 = p.ut.row0[u], nb = sl_len(kv, b);
    const int nr = p.ut.nrow[u];
    const int j0 = chunk * CH;
    // a chunk wholly past n_b has nothing to produce: its statistics and
    // logits are never read (rows_lse and the finalizers stop at n_b)
    if (j0 >= nb) return;
    const bool paged = kv.page_size != 0;
    // the page ids are loaded once, with Q, so no K load waits for a
    // page-table load of its own
    if (paged)
        for (int i = tid; i < CH / 16; i += 256) {
            const int pi = (j0 >> 4) + i;
            pgs[i] = pi < kv.max_pages ? kv.page_table[(int64_t)b * kv.max_pages + pi] : -1;
        }

    for (int e = tid; e < nr * D; e += 256) {
        const int r = e / D, d = e - (e / D) * D;
        const char *qp = p.q + ((int64_t)b * p.q_bstride + p.qoff[row0 + r] + d) * ESZ;
        qs[r][d] = F32 ? *(const float *)qp : bf16_bits_to_f32(*(const uint16_t *)qp);
    }
    __syncthreads();

    const int grp = tid / LPI, sl = tid - (tid / LPI) * LPI;
    // This lane's slice of every query row, in registers (the dot products
    // then read no LDS), and the dot product's sum over the LPI lanes of a
    // position with DPP row rotations when a position is one 16-lane row.
    float qr[8][EPL];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int i = 0; i < EPL; ++i) qr[r][i] = r < nr ? qs[r][sl * EPL + i] : 0.f;
    auto lane_sum = [&](float v) {
        if constexpr (LPI == 16) {
            return lane16_sum(v);
        } else if constexpr (LPI == 32) {
            v = lane16_sum(v);
            return v + __shfl_xor(v, 16, 64);
        } else {
#pragma unroll
            for (int o = LPI / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
            return v;
        }
    };
    // All of a lane's slice loads of a batch are issued before any is used.
    constexpr int NP = CH / IPP;              // positions per lane group
    constexpr int NB = NP < 8 ? NP : 8;       // positions per batch
    static_assert(NP % NB == 0, "batches");
#pragma unroll 1
    for (int t0 = 0; t0 < NP; t0 += NB) {
        u32x4 raw[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int pos = grp + (t0 + t) * IPP;
            const int j = j0 + pos;
            const char *row = nullptr;
            if (j < nb) {
                if (paged) {
                    const int pg = pgs[pos >> 4];
                    if (pg >= 0 && pg < kv.num_pages)
                        row = kv.k + ((((int64_t)pg * 16 + (j & 15)) * kv.Hkv + kvh) * D) * ESZ;
                } else {
                    row = kv.k + ((((int64_t)b * kv.N_max + j) * kv.Hkv + kvh) * D) * ESZ;
                }
            }
            raw[t] = row ? ld_stream16(row + sl * 16) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int pos = grp + (t0 + t) * IPP;
            const bool ok = j0 + pos < nb;
            float x[8];
            if constexpr (F32) {
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(raw[t][i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = __uint_as_float(raw[t][i] << 16);
                    x[2 * i + 1] = __uint_as_float(raw[t][i] & 0xffff0000u);
                }
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r < nr) {
                    float sdot = 0.f;
#pragma unroll
                    for (int i = 0; i < EPL; ++i) sdot += qr[r][i] * x[i];
                    sdot = lane_sum(sdot);
                    if (sl == 0) lg[r][pos] = ok ? sdot * p.scale_log2 : kNegInf;
                }
            }
        }
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    for (int r = wave; r < nr; r += 4) {
        float v[CH / 64];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) {
            v[i] = lg[r][lane + 64 * i];
            mx = fmaxf(mx, v[i]);
        }
        mx = wave_max(mx);
        const float muse = (mx == kNegInf) ? 0.f : mx;
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) z += exp2f(v[i] - muse);
        z = wave_sum(z);
        if (lane == 0) {
            float *st = p.stat + (((int64_t)b * p.total_rows + row0 + r) * p.nchunk + chunk) * 2;
            st[0] = mx;
            st[1] = z;
        }
        if (p.logit) {
            float *lp = p.logit + ((int64_t)b * p.total_rows + row0 + r) * p.N_max + j0;
#pragma unroll
            for (int i = 0; i < CH / 64; ++i) {
                const int pos = lane + 64 * i;
                if (j0 + pos < p.N_max) lp[pos] = v[i];
            }
        }
    }
}

// Target statistics, whole-row form: when the scored rows of one layer use
// every one of its KV heads (each KV head one unit of <= 8 rows), all of the
// layer's key bytes are needed, so a work-group streams whole position rows
// ([H_kv][128] bf16, contiguous) once instead of each head's 256-byte slices
// at the row stride in separate work-groups.  Lane t of a position's
// H_kv * 16 lanes holds 16 bytes of head (t / 16); a head's dot products are
// summed over its 16 lanes with DPP rotations.  Same outputs as
// unit_stats_valu: per-chunk (max, sum of exp2) per row, and the logits.
struct RowStatsParams {
    KvView kv;
    const char *q;                   // [B][S][128] bf16
    int32_t S;
    int32_t unit_of_head[16];        // unit index of each KV head
    int32_t row0[16], nrow[16];      // per unit
    float scale_log2;
    float *stat;                     // [B][S][nchunk][2]
    float *logit;                    // [B][S][N_max]
    int32_t nchunk, N_max;
};

template <int NR>   // rows per unit at most (1, 2, 4 or 8)
__global__ __launch_bounds__(256) void unit_stats_rows(RowStatsParams p) {
    constexpr int D = 128, EPL = 8;
    // loads in flight per lane: 8 (16, with fewer waves per SIMD, measured 2%
    // slower, 24 5% slower, 4 3% slower on the paged c5 cache)
    constexpr int NB = 8;
    extern __shared__ float lg[];    // [S][CH]
    __shared__ int pgs[CH / 16];
    const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const KvView &kv = p.kv;
    const int nb = sl_len(kv, b);
    const int j0 = chunk * CH;
    if (j0 >= nb) return;   // statistics and logits past n_b are never read
    const int LPP = kv.Hkv * 16;     // lanes per position (<= 256, a power of two)
    const int PPI = 256 / LPP;       // positions per load instruction
    const int g = (tid % LPP) >> 4, sl = tid & 15, pq = tid / LPP;
    const bool paged = kv.page_size != 0;
    if (paged)
        for (int i = tid; i < CH / 16; i += 256) {
            const int pi = (j0 >> 4) + i;
            pgs[i] = pi < kv.max_pages ? kv.page_table[(int64_t)b * kv.max_pages + pi] : -1;
        }
    const int u = p.unit_of_head[g];
    const int r0 = p.row0[u], nr = p.nrow[u];
    float qr[NR][EPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        u32x4 raw = u32x4{0u, 0u, 0u, 0u};
        if (r < nr) raw = *(const u32x4 *)(p.q + (((int64_t)b * p.S + r0 + r) * D + sl * EPL) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qr[r][2 * i] = __uint_as_float(raw[i] << 16);
            qr[r][2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
        }
    }
    __syncthreads();   // page ids in LDS
    const int64_t rowb = (int64_t)kv.Hkv * D * 2;   // bytes per position row
    const int NP = CH / PPI;                          // positions per lane
    for (int t0 = 0; t0 < NP; t0 += NB) {
        u32x4 raw[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int pos = pq + (t0 + t) * PPI;
            const int j = j0 + pos;
            const char *row = nullptr;
            if (t0 + t < NP && j < nb) {
                if (paged) {
                    const int pg = pgs[pos >> 4];
                    if (pg >= 0 && pg < kv.num_pages) row = kv.k + ((int64_t)pg * 16 + (j & 15)) * rowb;
                } else {
                    row = kv.k + ((int64_t)b * kv.N_max + j) * rowb;
                }
            }
            raw[t] = row ? ld_stream16(row + (g * 16 + sl) * 16) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            if (t0 + t >= NP) break;
            const int pos = pq + (t0 + t) * PPI;
            const bool ok = j0 + pos < nb;
            float x[EPL];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __uint_as_float(raw[t][i] << 16);
                x[2 * i + 1] = __uint_as_float(raw[t][i] & 0xffff0000u);
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (r < nr) {   // the same for the 16 lanes of a head
                    float sdot = 0.f;
#pragma unroll
                    for (int i = 0; i < EPL; ++i) sdot += qr[r][i] * x[i];
                    sdot = lane16_sum(sdot);
                    if (sl == 0) lg[(r0 + r) * CH + pos] = ok ? sdot * p.scale_log2 : kNegInf;
                }
            }
        }
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    for (int r = wave; r < p.S; r += 4) {
        float v[CH / 64];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) {
            v[i] = lg[r * CH + lane + 64 * i];
            mx = fmaxf(mx, v[i]);
        }
        mx = wave_max(mx);
        const float muse = (mx == kNegInf) ? 0.f : mx;
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) z += exp2f(v[i] - muse);
        z = wave_sum(z);
        if (lane == 0) {
            float *st = p.stat + (((int64_t)b * p.S + r) * p.nchunk + chunk) * 2;
            st[0] = mx;
            st[1] = z;
        }
        float *lp = p.logit + ((int64_t)b * p.S + r) * p.N_max + j0;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) {
            const int pos = lane + 64 * i;
            if (j0 + pos < p.N_max) lp[pos] = v[i];
        }
    }
}

// The whole-row form on the matrix cores, for units of five to eight rows
// (every head of a layer scored: the all-heads estimator, the per-head rows
// of the configuration search), where the VALU form's 16-lane sum per row
// and position bounds it.  A work-group takes the heads [z * HPG, (z + 1) *
// HPG) of its chunk (HPG = Hkv when the chunks alone fill the chip); wave w
// takes HPW of them and every subtile (HPG >= 4), or one head and every
// wph-th subtile (HPG < 4, wph = 4 / HPG).  The logits of one head's 16
// positions are one MFMA chain: A = the unit's query rows (padded to 16),
// B = the 16 key rows, d contracted in four 32-wide steps.  Key rows of
// positions past n_b or in absent pages are zero (logit 0, then masked past
// n_b), as in the VALU form.  The logits go to LDS, slot (local head, row)
// with a row stride of CH + 4 floats (the four lane groups of an MFMA
// result land in different banks), then one wave per slot writes the
// chunk statistics and the logit row, as the VALU form does.
constexpr int kRowsMfmaLdsStride = CH + 4;

template <int HPW>
__global__ __launch_bounds__(256, 2) void unit_stats_rows_mfma(RowStatsParams p, int HPG, int wph) {
    constexpr int D = 128, KK = 4, NSUB = CH / 16;
    extern __shared__ float lg[];    // [HPG][8][kRowsMfmaLdsStride]
    __shared__ int pgs[NSUB];
    const int chunk = blockIdx.x, b = blockIdx.y, hz = blockIdx.z, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const KvView &kv = p.kv;
    const int nb = sl_len(kv, b);
    const int j0 = chunk * CH;
    if (j0 >= nb) return;   // statistics and logits past n_b are never read
    const bool paged = kv.page_size != 0;
    if (paged && tid < NSUB) {
        const int pi = (j0 >> 4) + tid;
        pgs[tid] = pi < kv.max_pages ? kv.page_table[(int64_t)b * kv.max_pages + pi] : -1;
    }
    const int hl0 = (wave / wph) * HPW;   // first local head of this wave
    const int sub0 = wave % wph;          // first subtile; then every wph-th
    // Q fragments of this wave's heads (row lane & 15 of the head's unit,
    // d slice kk * 32 + (lane >> 4) * 8); padding rows are zero.
    bf16x8 qf[HPW][KK];
    int rbase[HPW], nrow[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const int u = p.unit_of_head[hz * HPG + hl0 + hh];
        rbase[hh] = p.row0[u];
        nrow[hh] = p.nrow[u];
        const int r = lane & 15;
        const bool ok = r < nrow[hh];
        const char *qp = p.q + (((int64_t)b * p.S + rbase[hh] + (ok ? r : 0)) * D + (lane >> 4) * 8) * 2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const u32x4 v = *(const u32x4 *)(qp + kk * 64);
            qf[hh][kk] = __builtin_bit_cast(bf16x8, ok ? v : u32x4{0u, 0u, 0u, 0u});
        }
    }
    __syncthreads();   // page ids in LDS
    const int64_t rowb = (int64_t)kv.Hkv * D * 2;   // bytes per position row
    const int gph = NSUB / wph / 4;                   // groups of 4 subtiles per head
    const int items = HPW * gph;
    // Key fragments of item `it` (local head it % HPW, subtile group
    // it / HPW: a wave's heads are read together, position by position);
    // every load of an item is issued; positions past n_b and absent pages
    // read row 0 and are zeroed after.
    auto load = [&](int it, u32x4 (&k)[4][KK], uint32_t &okm) {
        if (it >= items) return;   // wave-uniform
        const int hh = it % HPW, g = it / HPW;
        const int h = hz * HPG + hl0 + hh;
        okm = 0;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int sub = sub0 + (g * 4 + st) * wph;
            const int j = j0 + sub * 16 + (lane & 15);
            int64_t r = -1;
            if (paged) {
                const int pg = pgs[sub];
                if (j < nb && pg >= 0 && pg < kv.num_pages) r = (int64_t)pg * 16 + (j & 15);
            } else if (j < nb) {
                r = (int64_t)b * kv.N_max + j;
            }
            okm |= (r >= 0 ? 1u : 0u) << st;
            const char *row = kv.k + (r >= 0 ? r : 0) * rowb + (int64_t)h * D * 2 + (lane >> 4) * 16;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) k[st][kk] = *(const u32x4 *)(row + kk * 64);
        }
    };
    auto fold = [&](int it, const u32x4 (&k)[4][KK], uint32_t okm) {
        if (it >= items) return;
        const int hh = it % HPW, g = it / HPW;
        bf16x8 qc[KK];
        int rb0 = 0, nr = 0;
#pragma unroll
        for (int c = 0; c < HPW; ++c)
            if (c == hh) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) qc[kk] = qf[c][kk];
                rb0 = c;
                nr = nrow[c];
            }
        float *slot = lg + ((hl0 + rb0) * 8) * kRowsMfmaLdsStride;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int sub = sub0 + (g * 4 + st) * wph;
            const int pos = sub * 16 + (lane & 15);
            const bool ok = (okm >> st) & 1u;
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const u32x4 kv4 = ok ? k[st][kk] : u32x4{0u, 0u, 0u, 0u};
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[kk], __builtin_bit_cast(bf16x8, kv4), sc, 0, 0, 0);
            }
            const bool live = j0 + pos < nb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (lane >> 4) * 4 + i;
                if (r < nr) slot[r * kRowsMfmaLdsStride + pos] = live ? sc[i] * p.scale_log2 : kNegInf;
            }
        }
    };
    u32x4 kA[4][KK], kB[4][KK];
    uint32_t okA = 0, okB = 0;
    load(0, kA, okA);
    for (int it = 0; it < items; it += 2) {
        load(it + 1, kB, okB);
        fold(it, kA, okA);
        load(it + 2, kA, okA);
        fold(it + 1, kB, okB);
    }
    __syncthreads();
    // one wave per (local head, row) slot
    for (int sidx = wave; sidx < HPG * 8; sidx += 4) {
        const int hl = sidx >> 3, rr = sidx & 7;
        const int u = p.unit_of_head[hz * HPG + hl];
        if (rr >= p.nrow[u]) continue;
        const int r = p.row0[u] + rr;
        const float *src = lg + sidx * kRowsMfmaLdsStride;
        float v[CH / 64];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) {
            v[i] = src[lane + 64 * i];
            mx = fmaxf(mx, v[i]);
        }
        mx = wave_max(mx);
        const float muse = (mx == kNegInf) ? 0.f : mx;
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) z += exp2f(v[i] - muse);
        z = wave_sum(z);
        if (lane == 0) {
            float *st = p.stat + (((int64_t)b * p.S + r) * p.nchunk + chunk) * 2;
            st[0] = mx;
            st[1] = z;
        }
        float *lp = p.logit + ((int64_t)b * p.S + r) * p.N_max + j0;
#pragma unroll
        for (int i = 0; i < CH / 64; ++i) {
            const int pos = lane + 64 * i;
            if (j0 + pos < p.N_max) lp[pos] = v[i];
        }
    }
}

// Row log-sum-exp (log2 domain) from the per-chunk statistics.
// One wave per row; rows are sequence-major (rows_per_b rows per sequence)
// and only the chunks holding positions below n_b are read (the statistics
// passes may leave the others unwritten).
__global__ __launch_bounds__(256) void rows_lse(const float *stat, float *lse, int nrows_total, int nchunk,
                                                const int32_t *seq_lens, int rows_per_b, int chunk, int N_max) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= nrows_total) return;
    const float *st = stat + (int64_t)row * nchunk * 2;
    constexpr int MAXP = 8;   // (max, sum) pairs per lane held in registers
    if (nchunk <= 64 * MAXP) {
        // every pair of the row is requested together with the length (the
        // ones past n_b are in bounds and then ignored): one round trip
        float2 v[MAXP];
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int c = lane + 64 * i;
            v[i] = c < nchunk ? *(const float2 *)(st + 2 * c) : float2{kNegInf, 0.f};
        }
        const int nb = min(max(seq_lens[row / rows_per_b], 0), N_max);
        const int nv = min(nchunk, (nb + chunk - 1) / chunk);
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < MAXP; ++i)
            if (lane + 64 * i < nv) mx = fmaxf(mx, v[i].x);
        mx = wave_max(mx);
        const float muse = (mx == kNegInf) ? 0.f : mx;
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < MAXP; ++i)
            if (lane + 64 * i < nv) z += v[i].y * exp2f(v[i].x - muse);
        z = wave_sum(z);
        if (lane == 0) lse[row] = (z > 0.f) ? muse + __log2f(z) : __builtin_huge_valf();
        return;
    }
    const int nb = min(max(seq_lens[row / rows_per_b], 0), N_max);
    const int nv = min(nchunk, (nb + chunk - 1) / chunk);
    float mx = kNegInf;
    for (int c = lane; c < nv; c += 64) mx = fmaxf(mx, st[2 * c]);
    mx = wave_max(mx);
    const float muse = (mx == kNegInf) ? 0.f : mx;
    float z = 0.f;
    for (int c = lane; c < nv; c += 64) z += st[2 * c + 1] * exp2f(st[2 * c] - muse);
    z = wave_sum(z);
    if (lane == 0) lse[row] = (z > 0.f) ? muse + __log2f(z) : __builtin_huge_valf();
}

// Row normalisers between the caller's layout ([B][L_d][gamma][H_d], natural
// log) and the draft passes' ([B][L_d * Hkv_d][rows], log2, row r = step *
// G_d + head mod G_d of KV head head / G_d).  An empty row is -inf outside and
// +inf inside (its terms are exp2(logit - inf) = 0); other non-finite inputs
// are taken as empty rows.
__device__ __forceinline__ int64_t draft_lse_slot(int64_t i, int L_d, int gamma, int H_d, int Hkv_d, int G_d) {
    const int h = (int)(i % H_d);
    const int64_t t = i / H_d;
    const int g = (int)(t % gamma);
    const int64_t bl = t / gamma;   // b * L_d + l
    return (bl * Hkv_d + h / G_d) * (int64_t)(gamma * G_d) + g * G_d + h % G_d;
}
__global__ __launch_bounds__(256) void draft_lse_import(const float *in, float *lse, int64_t n, int L_d, int gamma,
                                                        int H_d, int Hkv_d, int G_d) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float v = in[i];
        lse[draft_lse_slot(i, L_d, gamma, H_d, Hkv_d, G_d)] = __builtin_isfinite(v) ? v * kLog2e : __builtin_huge_valf();
    }
}
__global__ __launch_bounds__(256) void draft_lse_export(const float *lse, float *out, int64_t n, int L_d, int gamma,
                                                        int H_d, int Hkv_d, int G_d) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float v = lse[draft_lse_slot(i, L_d, gamma, H_d, Hkv_d, G_d)];
        out[i] = __builtin_isfinite(v) ? v * kLn2 : kNegInf;
    }
}

// S_Target[b][j] = sum_r exp2(logit[r][j] - lse[r]).
// V4: four positions per lane (N_max % 4 == 0, so every logit row is
// 16-byte aligned); rows are summed in order either way.
template <bool V4>
__global__ __launch_bounds__(256) void target_finalize(const float *logit, const float *lse, float *out,
                                                       const int32_t *seq_lens, int S, int N_max) {
    const int b = blockIdx.y;
    const int nb = min(max(seq_lens[b], 0), N_max);
    if constexpr (V4) {
        const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
        if (j >= N_max) return;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (j < nb) {
            const float *lg = logit + (int64_t)b * S * N_max + j;
            const float *ls = lse + (int64_t)b * S;
#pragma unroll 8
            for (int r = 0; r < S; ++r) {
                const f32x4 v = *(const f32x4 *)(lg + (int64_t)r * N_max);
                const float m = ls[r];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += exp2f(v[i] - m);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (j + i >= nb) acc[i] = 0.f;
        }
        *(f32x4 *)(out + (int64_t)b * N_max + j) = acc;
    } else {
        const int j = blockIdx.x * 256 + threadIdx.x;
        if (j >= N_max) return;
        float acc = 0.f;
        if (j < nb) {
            for (int r = 0; r < S; ++r)
                acc += exp2f(logit[((int64_t)b * S + r) * N_max + j] - lse[(int64_t)b * S + r]);
        }
        out[(int64_t)b * N_max + j] = acc;
    }
}

// Per-row form: out[r][b][j] = exp2(logit[b][r][j] - lse[b][r]) for j < n_b, 0 beyond
// (V4: four positions per lane, N_max % 4 == 0).
template <bool V4>
__global__ __launch_bounds__(256) void target_rows_finalize(const float *logit, const float *lse, float *out,
                                                            const int32_t *seq_lens, int B, int S, int N_max) {
    const int b = blockIdx.y, r = blockIdx.z;
    const int nb = min(max(seq_lens[b], 0), N_max);
    const int64_t row = (int64_t)b * S + r;
    if constexpr (V4) {
        const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
        if (j >= N_max) return;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (j < nb) {
            const f32x4 x = *(const f32x4 *)(logit + row * N_max + j);
            const float m = lse[row];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (j + i < nb) ? exp2f(x[i] - m) : 0.f;
        }
        *(f32x4 *)(out + ((int64_t)r * B + b) * N_max + j) = v;
    } else {
        const int j = blockIdx.x * 256 + threadIdx.x;
        if (j >= N_max) return;
        out[((int64_t)r * B + b) * N_max + j] = (j < nb) ? exp2f(logit[row * N_max + j] - lse[row]) : 0.f;
    }
}

// ---------------------------------------------------------------------------
// Draft side, float32 storage: VALU accumulation pass.  One work-group per
// (sequence, chunk); loops over every unit in order.
template <int D, int NV>
struct DraftValuAccParams {
    KvView kv[NV];
    UnitTable ut;
    const char *q;
    int64_t q_bstride;
    int32_t qoff[kMaxScoreQoff];
    int32_t total_rows;
    float scale_log2;
    const float *lse;                // [B][total_rows]
    float *out;                      // [B][N_max]
    int32_t N_max;
};

template <int D, int NV>
__global__ __launch_bounds__(256) void draft_acc_valu(DraftValuAccParams<D, NV> p) {
    constexpr int LPI = D * 4 / 16;
    constexpr int IPP = 256 / LPI;
    __shared__ float qs[8][D];
    __shared__ float ls[8];
    __shared__ float acc[CH];
    const int chunk = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int j0 = chunk * CH;
    const int grp = tid / LPI, sl = tid - (tid / LPI) * LPI;
    for (int i = tid; i < CH; i += 256) acc[i] = 0.f;
    for (int u = 0; u < p.ut.n_units; ++u) {
        const KvView &kv = p.kv[p.ut.view[u]];
        const int kvh = p.ut.kvh[u], row0 = p.ut.row0[u], nr = p.ut.nrow[u];
        const int nb = sl_len(kv, b);
        __syncthreads();
        for (int e = tid; e < nr * D; e += 256) {
            const int r = e / D, d = e - (e / D) * D;
            qs[r][d] = *(const float *)(p.q + ((int64_t)b * p.q_bstride + p.qoff[row0 + r] + d) * 4);
        }
        if (tid < nr) ls[tid] = p.lse[(int64_t)b * p.total_rows + row0 + tid];
        __syncthreads();
        for (int pos = grp; pos < CH; pos += IPP) {
            const int j = j0 + pos;
            const bool ok = j < nb;
            float x[8];
            load_slice<true>(ok ? krow(kv, b, j, kvh, 4) : nullptr, sl, x);
            float tot = 0.f;
            for (int r = 0; r < nr; ++r) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) s += qs[r][sl * 4 + i] * x[i];
#pragma unroll
                for (int o = LPI / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
                tot += exp2f(s * p.scale_log2 - ls[r]);
            }
            if (sl == 0 && ok) acc[pos] += tot;
        }
    }
    __syncthreads();
    for (int i = tid; i < CH; i += 256) {
        const int j = j0 + i;
        if (j < p.N_max) p.out[(int64_t)b * p.N_max + j] = acc[i];
    }
}

// ---------------------------------------------------------------------------
// Draft side, bfloat16 storage: MFMA passes.  For unit u = (layer l, draft KV
// head c) the R = gamma * G_d rows are (step g, head c*G_d + hh), row index
// g * G_d + hh.  S = Q . K^T per 16-token subtile with
// v_mfma_f32_16x16x32_bf16: lane holds token (lane & 15) and rows
// rb*16 + (lane >> 4)*4 + i.

template <int D, int RB>
struct DraftMfma {
    static constexpr int KK = D / 32;

    // Q operand fragments of unit (l, c): row rb*16 + (lane&15), d slice kk*32 + (lane>>4)*8.
    // Branch-free: padding rows load row 0 and are zeroed by a select, so
    // every lane issues the same loads and the compiler can count them (a
    // load skipped on some paths makes every later wait a full drain).
    static __device__ __forceinline__ void load_q(const DraftScoreArgs &a, int b, int l, int c, int lane,
                                                  bf16x8 (&qf)[RB][KK]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rb * 16 + (lane & 15);
            const bool ok = r < a.rows;
            const int rr = ok ? r : 0;
            const int gs = rr / a.G_d, hh = rr - (rr / a.G_d) * a.G_d;
            const int64_t qbs = a.q_bstride ? a.q_bstride : (int64_t)a.L_d * a.gamma * a.H_d * D;
            const int64_t qss = a.q_sstride ? a.q_sstride : (int64_t)a.H_d * D;
            const uint16_t *qp = (const uint16_t *)a.q_draft + (int64_t)b * qbs + gs * qss +
                ((int64_t)l * a.gamma * a.H_d + c * a.G_d + hh) * D + (lane >> 4) * 8;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const u32x4 v = *(const u32x4 *)(qp + kk * 32);
                qf[rb][kk] = __builtin_bit_cast(bf16x8, ok ? v : u32x4{0u, 0u, 0u, 0u});
            }
        }
    }

    // K^T operand fragments of 4 subtiles (64 positions from j_base).  For a
    // contiguous cache the loads are branch-free (positions past n_b read a
    // valid row and are masked by the caller); a paged cache looks the page
    // up first.
    static __device__ __forceinline__ void load_k(const KvView &kv, int b, int c, int j_base, int nb, int lane,
                                                  bf16x8 (&kf)[4][KK]) {
        if (kv.page_size == 0) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int j = j_base + st * 16 + (lane & 15);
                const int jj = (j < nb) ? j : 0;
                const char *row = kv.k + ((((int64_t)b * kv.N_max + jj) * kv.Hkv + c) * D) * 2;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    kf[st][kk] = *(const bf16x8 *)(row + (kk * 32 + (lane >> 4) * 8) * 2);
            }
            return;
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int j = j_base + st * 16 + (lane & 15);
            const char *row = (j < nb) ? krow(kv, b, j, c, 2) : nullptr;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if (row) {
                    kf[st][kk] = *(const bf16x8 *)(row + (kk * 32 + (lane >> 4) * 8) * 2);
                } else {
                    for (int i = 0; i < 8; ++i) kf[st][kk][i] = (__bf16)0.f;
                }
            }
        }
    }

    // The same for a paged cache whose four page ids (one per 16-position
    // subtile, uniform across the wave) are already in registers: no
    // page-table load on the way to the K rows.
    static __device__ __forceinline__ void load_k_pg(const KvView &kv, const int (&pg)[4], int c, int j_base, int nb,
                                                     int lane, bf16x8 (&kf)[4][KK]) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int j = j_base + st * 16 + (lane & 15);
            const bool ok = j < nb && pg[st] >= 0 && pg[st] < kv.num_pages;
            const char *row = kv.k + ((((int64_t)(ok ? pg[st] : 0) * 16 + (j & 15)) * kv.Hkv + c) * D) * 2;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if (ok) {
                    kf[st][kk] = *(const bf16x8 *)(row + (kk * 32 + (lane >> 4) * 8) * 2);
                } else {
                    for (int i = 0; i < 8; ++i) kf[st][kk][i] = (__bf16)0.f;
                }
            }
        }
    }

    static __device__ __forceinline__ void logits(const bf16x8 (&qf)[RB][KK], const bf16x8 (&kf)[4][KK],
                                                  f32x4 (&s)[4][RB]) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[rb][kk], kf[st][kk], acc, 0, 0, 0);
                s[st][rb] = acc;
            }
    }
};

// Statistics pass.  Persistent work-groups walk the items (b, unit u,
// 4096-position chunk) round robin; each wave streams 1024 positions in
// groups of four 16-position subtiles, the next group's K fragments in
// flight while the current group is reduced into per-lane running
// (max, sum of exp2) pairs.  The first group (and the Q fragments) of the
// work-group's next item are requested during the last group of the
// current one, so the stream does not stall between items.
constexpr int kDraftStatChunk = 4096;
constexpr int kDraftStatMaxB = kMaxDraftBatch;   // sequences per call of the statistics pass

template <int D, int RB>
__global__ __launch_bounds__(256, (RB >= 3 || (D == 128 && RB >= 2)) ? 1 : 2) void draft_stats_mfma(DraftScoreArgs a) {
    using M = DraftMfma<D, RB>;
    __shared__ float red[4][RB * 16][2];
    __shared__ int pref[kDraftStatMaxB + 1];  // chunks below n_b of sequences before b
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int U = a.L_d * a.Hkv_d;
    const int nch = a.nchunk;                 // kDraftStatChunk-position chunks
    const int B = a.kv[0].B;
    constexpr int NG = kDraftStatChunk / 4 / 64;   // 64-position groups per wave
    static_assert(NG % 2 == 0, "groups are folded in pairs");
    // Items are (b, u, c) over the chunks that hold positions below n_b only
    // (a ragged batch skips the rest), numbered sequence by sequence: the
    // prefix of per-sequence chunk counts is built in LDS (B <= 1024, checked
    // by the launcher).
    for (int bb = threadIdx.x; bb < B; bb += blockDim.x)
        pref[bb + 1] = (sl_len(a.kv[0], bb) + kDraftStatChunk - 1) / kDraftStatChunk;
    __syncthreads();
    if (threadIdx.x == 0) {
        pref[0] = 0;
        for (int bb = 0; bb < B; ++bb) pref[bb + 1] += pref[bb];
    }
    __syncthreads();
    const int items = U * pref[B];
    struct Item { int b, u, c, l, kvh, nb, jw; };
    auto decode = [&](int it) {
        Item x;
        const int cu = it / U;                // chunk index over all sequences
        int lo = 0, hi = B - 1;               // the b with pref[b] <= cu < pref[b + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pref[mid] <= cu) lo = mid;
            else hi = mid - 1;
        }
        x.b = lo;
        const int nbc = pref[lo + 1] - pref[lo];
        const int r = it - U * pref[lo];      // within the sequence: u-major
        x.u = r / nbc;
        x.c = r - x.u * nbc;
        x.l = x.u / a.Hkv_d;
        x.kvh = x.u - x.l * a.Hkv_d;
        x.nb = sl_len(a.kv[x.l], x.b);
        x.jw = x.c * kDraftStatChunk + wave * (kDraftStatChunk / 4);
        return x;
    };
    int it = blockIdx.x;
    if (it >= items) return;
    // Paged caches: lane t holds the page id of the wave's t-th 16-position
    // page (a wave spans kDraftStatChunk / 4 = 1024 positions = 64 pages), so
    // the K loads of a group need no page-table load first; the next item's
    // ids are loaded when the current item starts.
    const bool paged = a.kv[0].page_size != 0;
    auto load_pg = [&](const Item &x) -> int {
        if (!paged) return 0;
        const KvView &kv = a.kv[x.l];
        const int pgi = (x.jw >> 4) + lane;
        return pgi < kv.max_pages ? kv.page_table[(int64_t)x.b * kv.max_pages + pgi] : -1;
    };
    auto load_kg = [&](const Item &x, int pgl, int gi, bf16x8 (&k)[4][M::KK]) {
        const int jbase = x.jw + gi * 64;
        if (paged) {
            int pg[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) pg[st] = __builtin_amdgcn_readlane(pgl, gi * 4 + st);
            M::load_k_pg(a.kv[x.l], pg, x.kvh, jbase, x.nb, lane, k);
        } else {
            M::load_k(a.kv[x.l], x.b, x.kvh, jbase, x.nb, lane, k);
        }
    };
    // two named operand sets keep the double buffer in registers
    bf16x8 qf[RB][M::KK], qn[RB][M::KK];
    bf16x8 kA[4][M::KK], kB[4][M::KK];
    Item cur = decode(it);
    int pg_cur = load_pg(cur);
    M::load_q(a, cur.b, cur.l, cur.kvh, lane, qf);
    load_kg(cur, pg_cur, 0, kA);
    for (; it < items; it += gridDim.x) {
        const int nxt_it = it + gridDim.x;
        const Item nxt = decode(nxt_it < items ? nxt_it : it);
        const int pg_nxt = load_pg(nxt);
        float mrun[RB][4], zrun[RB][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mrun[rb][i] = kNegInf;
                zrun[rb][i] = 0.f;
            }
        auto fold = [&](int gi, const bf16x8 (&k)[4][M::KK]) {
            f32x4 sc[4][RB];
            M::logits(qf, k, sc);
            const int jg = cur.jw + gi * 64;
            const bool full = jg + 64 <= cur.nb;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float mx = mrun[rb][i];
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        float v = sc[st][rb][i] * a.scale_log2;
                        if (!full && jg + st * 16 + (lane & 15) >= cur.nb) v = kNegInf;
                        sc[st][rb][i] = v;
                        mx = fmaxf(mx, v);
                    }
                    const float mu = (mx == kNegInf) ? 0.f : mx;
                    float z = zrun[rb][i] * __builtin_amdgcn_exp2f(mrun[rb][i] - mu);
#pragma unroll
                    for (int st = 0; st < 4; ++st) z += __builtin_amdgcn_exp2f(sc[st][rb][i] - mu);
                    mrun[rb][i] = mx;
                    zrun[rb][i] = z;
                }
        };
#pragma unroll 1
        for (int gi = 0; gi < NG; gi += 2) {
            load_kg(cur, pg_cur, gi + 1, kB);
            fold(gi, kA);
            if (gi + 2 < NG) {
                load_kg(cur, pg_cur, gi + 2, kA);
            } else if (nxt_it < items) {   // prefetch the next item's first group
                M::load_q(a, nxt.b, nxt.l, nxt.kvh, lane, qn);
                load_kg(nxt, pg_nxt, 0, kA);
            }
            fold(gi + 1, kB);
        }
        // combine the 16 token lanes of each row, then the four waves
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mx = lane16_max(mrun[rb][i]);
                const float mu = (mx == kNegInf) ? 0.f : mx;
                const float z = lane16_sum(zrun[rb][i] * __builtin_amdgcn_exp2f(mrun[rb][i] - mu));
                if ((lane & 15) == 0) {
                    const int r = rb * 16 + (lane >> 4) * 4 + i;
                    red[wave][r][0] = mx;
                    red[wave][r][1] = z;
                }
            }
        lds_barrier();   // the prefetch above stays in flight
        if (threadIdx.x < a.rows) {
            const int r = threadIdx.x;
            float mx = kNegInf;
#pragma unroll
            for (int w = 0; w < 4; ++w) mx = fmaxf(mx, red[w][r][0]);
            const float mu = (mx == kNegInf) ? 0.f : mx;
            float z = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) z += red[w][r][1] * __builtin_amdgcn_exp2f(red[w][r][0] - mu);
            float *st = a.stat + ((((int64_t)cur.b * U + cur.u) * a.rows + r) * nch + cur.c) * 2;
            st[0] = mx;
            st[1] = z;
        }
        lds_barrier();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int kk = 0; kk < M::KK; ++kk) qf[rb][kk] = qn[rb][kk];
        cur = nxt;
        pg_cur = pg_nxt;
    }
}

// Accumulation pass.  Persistent work-groups walk the items (b, 256-position
// chunk); each wave owns 64 positions and loops over every draft unit in a
// fixed order, the next unit's operands in flight, so S_Draft is summed in
// registers without atomics.
//
// W > 0 is the per-step form used for the window attention A of Eq. (1)
// (one layer, the window queries as the "draft" rows, which are step-major
// within a unit): instead of one sum over all rows, lane sums are kept per
// step (step = row / G_d, at most W steps) and written, times steps_scale
// (1 / H_q: the head mean), to steps_out [B][gamma][N_max].  SA (G_d a
// multiple of 4): the four rows a lane holds per row block, rows
// rb * 16 + (lane >> 4) * 4 + i, share one step, so their four terms are
// summed before the one per-step select.
constexpr int kDraftAccChunk = 256;

template <int D, int RB, bool PAGED, int W = 0, bool SA = false>
__global__ __launch_bounds__(256, ((D == 128 && RB >= 2) || (W > 0 && RB >= 4)) ? 1 : 2) void draft_acc_mfma(DraftScoreArgs a) {
    using M = DraftMfma<D, RB>;
    constexpr int KK = M::KK;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int U = a.L_d * a.Hkv_d;
    const KvView &k0 = a.kv[0];   // every draft layer has this geometry (checked on the host)
    const int N = k0.N_max;
    const int B = k0.B;
    const int64_t sbs = a.steps_bstride ? a.steps_bstride : a.gamma;   // steps_out rows per sequence
    const int64_t sss = a.steps_sstride ? a.steps_sstride : 1;         // and between steps
    // Items are (b, chunk) over the chunks that hold positions below n_b
    // only, numbered sequence by sequence (B <= kDraftStatMaxB, checked by
    // the launchers), so a ragged batch spreads evenly over the groups; the
    // chunks wholly past n_b are zero-filled first.
    __shared__ int pref[kDraftStatMaxB + 1];
    for (int bb = threadIdx.x; bb < B; bb += blockDim.x)
        pref[bb + 1] = (sl_len(k0, bb) + kDraftAccChunk - 1) / kDraftAccChunk;
    __syncthreads();
    if (threadIdx.x == 0) {
        pref[0] = 0;
        for (int bb = 0; bb < B; ++bb) pref[bb + 1] += pref[bb];
    }
    __syncthreads();
    const int items = pref[B];
    for (int bb = 0; bb < B; ++bb) {
        const int j0 = (pref[bb + 1] - pref[bb]) * kDraftAccChunk;
        for (int j = j0 + blockIdx.x * 256 + (int)threadIdx.x; j < N; j += gridDim.x * 256) {
            if constexpr (W > 0) {
                for (int q2 = 0; q2 < a.gamma; ++q2) a.steps_out[((int64_t)bb * sbs + q2 * sss) * N + j] = 0.f;
            } else {
                a.s_draft[(int64_t)bb * N + j] = 0.f;
            }
        }
    }
    // per-lane parts of the Q addresses (row rb*16 + (lane & 15)) and of the
    // normaliser index (rows rb*16 + (lane >> 4)*4 + i); padding rows read
    // row 0 and are masked
    int qoff[RB];
    bool qok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rb * 16 + (lane & 15);
        qok[rb] = r < a.rows;
        const int rr = qok[rb] ? r : 0;
        const int qss = a.q_sstride ? (int)a.q_sstride : a.H_d * D;   // < 2^31 / 4 (checked on the host)
        qoff[rb] = (rr / a.G_d) * qss + (rr - (rr / a.G_d) * a.G_d) * D + (lane >> 4) * 8;
    }
    // step of each of this lane's result rows (rows past the last are masked
    // by an infinite normaliser; their step is clamped)
    int rstep[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb * 16 + (lane >> 4) * 4 + i;
            rstep[rb][i] = W > 0 ? min(r / a.G_d, W - 1) : 0;
        }
    constexpr int NS = W > 0 ? W : 1;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        int lo = 0, hi = B - 1;   // the b with pref[b] <= it < pref[b + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pref[mid] <= it) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo, c = it - pref[lo];
        const int jb = c * kDraftAccChunk + wave * 64;
        const int nb = sl_len(k0, b);
        if (jb >= nb) {   // this wave's positions are all past the sequence: zeros, no work
            const int j = jb + lane;
            if (j < N) {
                if constexpr (W > 0) {
                    for (int q2 = 0; q2 < a.gamma; ++q2) a.steps_out[((int64_t)b * sbs + q2 * sss) * N + j] = 0.f;
                } else {
                    a.s_draft[(int64_t)b * N + j] = 0.f;
                }
            }
            continue;
        }
        const float *lse_b = a.lse + (int64_t)b * U * a.rows;
        float acc[4][NS];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int q = 0; q < NS; ++q) acc[st][q] = 0.f;
        // byte offset of this lane's K row in a layer, per subtile (positions
        // past n_b read row 0 of the sequence and are masked)
        int64_t koff[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int j = jb + st * 16 + (lane & 15);
            koff[st] = (((int64_t)b * N + (j < nb ? j : 0)) * k0.Hkv * D + (lane >> 4) * 8) * 2;
        }
        // Operands in two named sets, one unit in flight while the other is
        // folded (a third set measured no faster).  Named sets stay in
        // registers; a runtime-indexed set would live in scratch memory.
        // Past the last unit the loads repeat the last unit (never folded),
        // so every load is unconditional and the compiler's waits stay exact.
        bf16x8 qA[RB][KK], qB[RB][KK];
        bf16x8 kA[4][KK], kB[4][KK];
        float lA[RB][4], lB[RB][4];
        // Paged: the page ids of this wave's 64 positions (4 pages) for every
        // draft layer, loaded once per item: lane 4 * (l % 16) + s holds page s
        // of layer l in pgA (l < 16) or pgB (l >= 16).  Loaded layer by layer
        // (uniform code), so the layer descriptors are never indexed per lane.
        int pgA = -1, pgB = -1;
        if constexpr (PAGED) {
            const int pidx = (jb >> 4) + (lane & 3);
#pragma unroll 1
            for (int l = 0; l < a.L_d; ++l) {
                const KvView &kv = a.kv[l];
                if ((lane >> 2) == (l & 15)) {
                    const int v = pidx < kv.max_pages ? kv.page_table[(int64_t)b * kv.max_pages + pidx] : -1;
                    if (l < 16) pgA = v;
                    else pgB = v;
                }
            }
        }
        auto load_k = [&](int u, bf16x8 (&k)[4][KK]) {
            u = (u < U) ? u : U - 1;
            const int l = u / a.Hkv_d, kvh = u - (u / a.Hkv_d) * a.Hkv_d;
            if constexpr (PAGED) {
                int pg[4];
                const int src = l < 16 ? pgA : pgB;
#pragma unroll
                for (int st = 0; st < 4; ++st) pg[st] = __builtin_amdgcn_readlane(src, (l & 15) * 4 + st);
                M::load_k_pg(a.kv[l], pg, kvh, jb, nb, lane, k);
            } else {
                const char *base = a.kv[l].k + (int64_t)kvh * D * 2;
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) k[st][kk] = *(const bf16x8 *)(base + koff[st] + kk * 64);
            }
        };
        auto load_ql = [&](int u, bf16x8 (&q)[RB][KK], float (&ls)[RB][4]) {
            u = (u < U) ? u : U - 1;
            const int l = u / a.Hkv_d, kvh = u - (u / a.Hkv_d) * a.Hkv_d;
            const int64_t qbs = a.q_bstride ? a.q_bstride : (int64_t)a.L_d * a.gamma * a.H_d * D;
            const uint16_t *qb = (const uint16_t *)a.q_draft + (int64_t)b * qbs +
                (((int64_t)l * a.gamma) * a.H_d + kvh * a.G_d) * D;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const u32x4 v = *(const u32x4 *)(qb + qoff[rb] + kk * 32);
                    q[rb][kk] = __builtin_bit_cast(bf16x8, qok[rb] ? v : u32x4{0u, 0u, 0u, 0u});
                }
            const float *lu = lse_b + (int64_t)u * a.rows;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rb * 16 + (lane >> 4) * 4 + i;
                    const float v = lu[r < a.rows ? r : 0];
                    ls[rb][i] = (r < a.rows) ? v : __builtin_huge_valf();
                }
        };
        auto fold_unit = [&](int u, const bf16x8 (&q)[RB][KK], const bf16x8 (&k)[4][KK], const float (&ls)[RB][4]) {
            if (u >= U) return;
#pragma unroll
            for (int st = 0; st < 4; ++st) {   // one subtile's logits live at a time
                float t[NS];
#pragma unroll
                for (int q2 = 0; q2 < NS; ++q2) t[q2] = 0.f;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[rb][kk], k[st][kk], sc, 0, 0, 0);
                    if constexpr (W > 0 && SA) {
                        float e4 = 0.f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) e4 += __builtin_amdgcn_exp2f(sc[i] * a.scale_log2 - ls[rb][i]);
#pragma unroll
                        for (int q2 = 0; q2 < NS; ++q2) t[q2] += (rstep[rb][0] == q2) ? e4 : 0.f;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float e = __builtin_amdgcn_exp2f(sc[i] * a.scale_log2 - ls[rb][i]);
                            if constexpr (W > 0) {
#pragma unroll
                                for (int q2 = 0; q2 < NS; ++q2) t[q2] += (rstep[rb][i] == q2) ? e : 0.f;
                            } else {
                                t[0] += e;
                            }
                        }
                    }
                }
                if (jb + st * 16 + (lane & 15) < nb) {
#pragma unroll
                    for (int q2 = 0; q2 < NS; ++q2) acc[st][q2] += t[q2];
                }
            }
        };
        load_k(0, kA);
        load_ql(0, qA, lA);
        for (int u = 0; u < U; u += 2) {
            load_ql(u + 1, qB, lB); load_k(u + 1, kB); fold_unit(u + 0, qA, kA, lA);
            load_ql(u + 2, qA, lA); load_k(u + 2, kA); fold_unit(u + 1, qB, kB, lB);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int j = jb + st * 16 + (lane & 15);
            if constexpr (W > 0) {
#pragma unroll
                for (int q2 = 0; q2 < NS; ++q2) {
                    const float v = group4_sum(acc[st][q2]);
                    if (lane < 16 && j < N && q2 < a.gamma)
                        a.steps_out[((int64_t)b * sbs + q2 * sss) * N + j] = v * a.steps_scale;
                }
            } else {
                const float v = group4_sum(acc[st][0]);
                if (lane < 16 && j < N) a.s_draft[(int64_t)b * N + j] = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Draft side, streaming form for bfloat16 drafts (contiguous or paged) with
// two 64-wide KV heads, where a draft layer's position row is 256 bytes
// ([2][64] bf16).
// Every wave streams its own positions through a private 16 KiB LDS ring of
// stages of one layer, fetched with the nontemporal global->LDS DMA (each
// row is read once per pass), while it computes on an earlier stage.  The
// sixteen 16-byte chunks of a position row are stored XOR-swizzled by the
// position's low four bits, so a K-operand read (16 positions, one chunk
// each) touches 16 distinct bank groups.  Register loads on the way (Q
// fragments, row normalisers, lengths) complete in order with the DMA, and
// every stage starts with a vmcnt wait that leaves only later stages in
// flight, so a stage never reads LDS before its own bytes have landed.
// Up to two row blocks per KV head: two 8 KiB stages of 32 full position
// rows (both KV heads, one stage in flight while the other is computed) and
// two 4-wave groups per CU.
//
// Three or four row blocks stream one KV head per item (HALF): stages hold
// 128-byte head halves, the operands of one head fit two groups per CU, and
// the two heads' accumulation results are partial sums added by
// draft_part_sum.  The statistics pass over half rows (DEEP) splits its ring
// into four 4 KiB stages of 32 positions, three in flight while one is
// computed; the accumulation pass keeps two 8 KiB stages of 64 positions,
// which measured faster there.  (A full-row form at one group per CU, with
// 64-position stages to keep the bytes in flight, had run no faster than the
// register-staged kernels, which now serve only the geometries neither
// streaming form covers.)
template <int RB, bool HALF = false, bool DEEP = false>
struct StreamGeom {
    static_assert(HALF || RB <= 2, "full-row streaming: at most two row blocks");
    static_assert(!DEEP || HALF, "four-stage rings: half rows only");
    static constexpr int RBY = HALF ? 128 : 256;      // stage bytes per position
    static constexpr int STAGE = DEEP ? 4096 : 8192;  // bytes per stage
    static constexpr int NSLOT = 16384 / STAGE;       // stages in a wave's ring
    static constexpr int POS = STAGE / RBY;           // positions per stage
    static constexpr int NI = STAGE / 1024;           // DMA instructions per stage
    static constexpr int NH = HALF ? 1 : 2;           // heads per item
    static constexpr int GROUPS = 512;                // persistent work-groups
};

// Wait until the stage about to be computed has landed, while the `ahead`
// stages issued after it (NI instructions each; ahead < A) stay in flight.
// Vector-memory loads complete in issue order, and any other request issued
// after that stage only makes the wait longer.
template <int A, int NI>
__device__ __forceinline__ void stream_wait(int ahead) {
    if constexpr (A <= 1) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= A - 1) wait_vmcnt<(A - 1) * NI>();
        else stream_wait<A - 1, NI>(ahead);
    }
}

// 16-byte chunk swizzle of stage row rho: full rows (16 chunks) by the low
// four bits; half rows (8 chunks, two rows per 256-byte bank span) by bits
// 1..3, so the 16 positions of a K-operand read hit 16 distinct bank groups.
template <bool HALF>
__device__ __forceinline__ int stream_swz(int rho) {
    return HALF ? ((rho >> 1) & 7) : (rho & 15);
}
constexpr int kStreamGroups = 512;

// DMA of the POS positions j0 .. j0 + POS - 1 of one layer into `stage` (32
// full rows, or 32 or 64 head halves when HALF); `seq` is the layer's k pointer
// advanced to the sequence.  Positions past the cache end read the last row
// (the caller masks them).
template <int POS, bool HALF>
__device__ __forceinline__ void stream_issue(const char *seq, int j0, int jlast, int hoff, int lane, uint8_t *stage) {
    constexpr int CPR = (HALF ? 128 : 256) / 16;   // chunks per stage row
    constexpr int PPI = 64 / CPR;                  // positions per instruction
#pragma unroll
    for (int i = 0; i < POS / PPI; ++i) {
        const int rho = i * PPI + lane / CPR;
        const int chunk = (lane % CPR) ^ stream_swz<HALF>(rho);
        const uint32_t j = (uint32_t)min(j0 + rho, jlast);
        dma16_stream(seq + (j * 256u + (uint32_t)hoff + (uint32_t)chunk * 16u), stage + i * 1024);
    }
}

// All-zero K row: the source of positions whose page id is out of range
// (they score as an all-zero key, as in the register-staged kernels).
__device__ __align__(256) uint8_t g_zero_krow[256] = {0};

// Paged form of stream_issue: stage s of a wave's span, whose POS / 16
// pages have their ids in lanes (POS / 16) s + 0, 1, .. of `pgv`; `pool` is
// the layer's k pointer (row r of the pool at r * 256 bytes).
template <int POS, bool HALF>
__device__ __forceinline__ void stream_issue_pg(const char *pool, int pgv, int s, int num_pages, int hoff, int lane,
                                                uint8_t *stage) {
    constexpr int NP = POS / 16;
    constexpr int CPR = (HALF ? 128 : 256) / 16;
    constexpr int PPI = 64 / CPR;
    int pgs[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) pgs[k] = __builtin_amdgcn_readlane(pgv, NP * s + k);
#pragma unroll
    for (int i = 0; i < POS / PPI; ++i) {
        const int rho = i * PPI + lane / CPR;   // on page rho / 16 of the stage
        const int chunk = (lane % CPR) ^ stream_swz<HALF>(rho);
        const int pg = pgs[(i * PPI) >> 4];
        const char *src = (pg >= 0 && pg < num_pages)
                              ? pool + (((int64_t)pg * 16 + (rho & 15)) * 256 + hoff + chunk * 16)
                              : (const char *)g_zero_krow + chunk * 16;
        dma16_stream(src, stage + i * 1024);
    }
}

// Page ids of the `npg` pages from position j0 on of sequence b, lane t
// holding page j0 / 16 + t (-1 past the table).
__device__ __forceinline__ int stream_load_pg(const KvView &kv, int b, int j0, int npg, int lane) {
    const int pi = (j0 >> 4) + lane;
    return (lane < npg && pi < kv.max_pages) ? kv.page_table[(int64_t)b * kv.max_pages + pi] : -1;
}

// Buffer resource over `bytes` bytes at `base` (loads past the end read 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane byte offsets of the Q fragments of a (sequence, draft layer)
// block [gamma][H_d][64]: row rb*16 + (lane & 15) of KV head 0 (head h adds
// h * G_d rows of 128 bytes), d slice (lane >> 4) * 8.  Padding rows read
// row 0: their logits are never used (the statistics pass does not store
// them; the accumulation pass gives them an infinite normaliser).
template <int RB>
__device__ __forceinline__ void stream_qoff(const DraftScoreArgs &a, int lane, uint32_t (&qo)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rb * 16 + (lane & 15);
        const int rr = r < a.rows ? r : 0;
        qo[rb] = (uint32_t)(((rr / a.G_d) * a.H_d + (rr - (rr / a.G_d) * a.G_d)) * 128 + (lane >> 4) * 16);
    }
}

// Q fragments of KV heads h0 .. h0 + NH - 1 of (sequence, draft layer).
template <int RB, int NH>
__device__ __forceinline__ void stream_load_q(const DraftScoreArgs &a, int b, int l, int h0, const uint32_t (&qo)[RB],
                                              bf16x8 (&q)[NH][RB][2]) {
    // (b, l, h0) are wave-uniform; saying so keeps the buffer resource in
    // scalar registers (otherwise each load becomes a per-lane loop)
    b = __builtin_amdgcn_readfirstlane(b);
    l = __builtin_amdgcn_readfirstlane(l);
    h0 = __builtin_amdgcn_readfirstlane(h0);
    const uint32_t blk = (uint32_t)(a.gamma * a.H_d * 128);
    const __amdgpu_buffer_rsrc_t r = stream_rsrc((const char *)a.q_draft + ((int64_t)b * a.L_d + l) * blk, blk);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                q[h][rb][kk] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, qo[rb] + kk * 64, (h0 + h) * a.G_d * 128, 0));
}

// K operand (head h, both k-steps) of 16-position subtile `st` of a stage:
// lane holds position st * 16 + (lane & 15), d slice kk * 32 + (lane >> 4) * 8.
template <bool HALF>
__device__ __forceinline__ void stream_kfrag(uint32_t base, int st, int h, int lane, bf16x8 (&k)[2]) {
    const int rho = st * 16 + (lane & 15);
    uint32_t ad[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int chunk = (HALF ? 0 : h * 8) + kk * 4 + (lane >> 4);
        ad[kk] = base + rho * (HALF ? 128 : 256) + ((chunk ^ stream_swz<HALF>(rho)) << 4);
    }
    u32x4 raw[2];
    ds_read_b128_n(ad, raw);
    k[0] = __builtin_bit_cast(bf16x8, raw[0]);
    k[1] = __builtin_bit_cast(bf16x8, raw[1]);
}

// Statistics pass, streaming form.  Items (b, layer, 4096-position chunk)
// walk round robin over the persistent groups; wave w streams positions
// w * 1024 .. + 1023 of the chunk (stages past n_b are skipped) keeping
// per-lane running (max, sum of exp2) pairs for its KV heads.  An item's
// first stage requests the next item's page ids and Q fragments, and its
// last stages issue the next item's first DMA stages, so the ring stays as
// full across items as inside one; items alternate between two named Q
// sets.  The cross-wave combine alternates between two LDS buffers, so one
// barrier per item suffices.
template <int RB, bool PAGED, bool HALF, int CHUNK = kDraftStatChunk>
__global__ __launch_bounds__(256, 2) void draft_stats_stream(DraftScoreArgs a) {
    // a paged wave span's page ids are one per lane: at most 64 pages
    static_assert(!PAGED || CHUNK / 4 / 16 <= 64, "paged items of at most 4096 positions");
    constexpr int KK = 2;
    using GM = StreamGeom<RB, HALF, HALF>;
    constexpr int POS = GM::POS;
    constexpr int NH = GM::NH;                 // heads per item (HALF: one, item.h)
    constexpr int NHI = HALF ? 2 : 1;          // items per (b, layer, chunk)
    constexpr int PER_WAVE = CHUNK / 4;
    constexpr int NSTAGE = PER_WAVE / POS;
    constexpr int NSL = GM::NSLOT;
    constexpr int AHEAD = NSL - 1;             // stages in flight beyond the one computed
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4][NSL][GM::STAGE];
    __shared__ float red[2][4][NH][RB * 16][2];
    __shared__ int pref[kDraftStatMaxB + 1];   // chunks below n_b of sequences before b
    __shared__ int slen[kDraftStatMaxB];       // n_b (every draft layer has layer 0's lengths)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int U = a.L_d * 2;
    const int nch = a.nchunk;
    const int B = a.kv[0].B;
    // Items are (b, layer, chunk) over the chunks that hold positions below
    // n_b only, numbered sequence by sequence (B <= kDraftStatMaxB, checked
    // by the launcher), so a ragged batch spreads evenly over the groups.
    for (int bb = threadIdx.x; bb < B; bb += blockDim.x) {
        const int n = sl_len(a.kv[0], bb);
        slen[bb] = n;
        pref[bb + 1] = (n + CHUNK - 1) / CHUNK;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        pref[0] = 0;
        for (int bb = 0; bb < B; ++bb) pref[bb + 1] += pref[bb];
    }
    __syncthreads();
    const int per = a.L_d * NHI;              // items per chunk of a sequence
    const int items = per * __builtin_amdgcn_readfirstlane(pref[B]);
    struct Item { int b, l, h, c, nb, jw, nst; const char *seq; int jlast; };
    auto decode = [&](int it) {
        Item x;
        const int cu = it / per;               // chunk index over all sequences
        int lo = 0, hi = B - 1;                // the b with pref[b] <= cu < pref[b + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (lds_read_i32(&pref[mid]) <= cu) lo = mid;
            else hi = mid - 1;
        }
        // every field is the same across the wave: readfirstlane makes that
        // visible to the compiler, so tests on them are scalar branches
        // (the LDS reads above otherwise make them look per-lane)
        x.b = __builtin_amdgcn_readfirstlane(lo);
        const int p0 = __builtin_amdgcn_readfirstlane(lds_read_i32(&pref[lo]));
        const int nbc = __builtin_amdgcn_readfirstlane(lds_read_i32(&pref[lo + 1])) - p0;
        const int r = it - per * p0;   // within the sequence: (layer, head)-major
        const int u = r / nbc;
        x.c = r - u * nbc;
        x.l = u / NHI;
        x.h = u - x.l * NHI;
        // from LDS: a global load here would be waited for together with
        // every stage already in flight
        x.nb = __builtin_amdgcn_readfirstlane(lds_read_i32(&slen[x.b]));
        x.jw = x.c * CHUNK + __builtin_amdgcn_readfirstlane(wave) * PER_WAVE;
        const int left = x.nb - x.jw;
        x.nst = left <= 0 ? 0 : min(NSTAGE, (left + POS - 1) / POS);
        x.seq = PAGED ? a.kv[x.l].k : a.kv[x.l].k + (int64_t)x.b * a.kv[x.l].N_max * 256;
        x.jlast = a.kv[x.l].N_max - 1;
        return x;
    };
    uint32_t qo[RB];
    stream_qoff<RB>(a, lane, qo);
    int slot = 0, islot = 0, par = 0;   // ring slots of the next stage to compute / to issue
    // paged caches: the page ids of an item's wave span (64 pages), one per lane
    auto load_pg = [&](const Item &x) -> int {
        return PAGED ? stream_load_pg(a.kv[x.l], x.b, x.jw, PER_WAVE / 16, lane) : 0;
    };
    auto issue = [&](const Item &x, int pgv, int s, uint8_t *stage) __attribute__((always_inline)) {
        if constexpr (PAGED) stream_issue_pg<POS, HALF>(x.seq, pgv, s, a.kv[x.l].num_pages, x.h * 128, lane, stage);
        else stream_issue<POS, HALF>(x.seq, x.jw + s * POS, x.jlast, x.h * 128, lane, stage);
    };
    // One item on Q set q (page ids pg), `ci` of whose stages were issued
    // before it began; requests the next item's Q into qn (page ids into
    // pgn) and keeps AHEAD stages in flight, running on into the next item's
    // first stages.  Returns how many of those it issued.
    auto item = [&](const Item &cur, const Item &nxt, bool has_next, const bf16x8 (&q)[NH][RB][KK],
                    bf16x8 (&qn)[NH][RB][KK], const int &pg, int &pgn, int ci) -> int {
        ci = __builtin_amdgcn_readfirstlane(ci);
        // Per lane and row: zrun = sum of exp2(v - mrun) over the lane's
        // positions so far, where mrun is a reference at least every such v
        // that moves only when a logit passes it, and then to that logit + 16:
        // most pairs of logits cost two exp2 and no rescale, terms stay <= 1,
        // and the reference is finite (-FLT_MAX for a lane with no valid
        // position in the item).
        float mrun[NH][RB][4], zrun[NH][RB][4];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    mrun[h][rb][i] = -kFltMax;
                    zrun[h][rb][i] = 0.f;
                }
        const int nn = has_next ? nxt.nst : 0;
        int ni = 0;   // stages of the next item issued
        // top up to AHEAD stages in flight after stage s (s = -1: none computed yet)
        auto top_up = [&](int s) __attribute__((always_inline)) {
            // (the counters move by arithmetic: incrementing one of two
            // through a selected reference had put both in scratch memory)
            while ((ci - 1 - s) + ni < AHEAD) {
                const bool own = ci < cur.nst;
                if (!own && ni >= nn) break;
                if (own) issue(cur, pg, ci, ring[wave][islot]);
                else issue(nxt, pgn, ni, ring[wave][islot]);
                ci += own ? 1 : 0;
                ni += own ? 0 : 1;
                islot = (islot + 1) & (NSL - 1);
            }
        };
        // FIRST: the item's first stage (its first pair sets the references);
        // a compile-time flag, so the other stages carry no trace of that path
        auto stage = [&](int s, auto first) {
            constexpr bool FIRST = decltype(first)::value;
            const uint32_t base = lds_addr(ring[wave][slot]);
            const int j0 = cur.jw + s * POS;
            const bool full = j0 + POS <= cur.nb;
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int pr = 0; pr < POS / 32; ++pr) {   // pairs of 16-position subtiles
                f32x4 sc[2][RB];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    bf16x8 k[2];
                    stream_kfrag<HALF>(base, pr * 2 + st, h, lane, k);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < KK; ++kk)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[h][rb][kk], k[kk], acc, 0, 0, 0);
                        sc[st][rb] = acc;
                    }
                }
                const float sl = a.scale_log2;
                // one wave-uniform test per pair (written inside the element
                // loops it became sixteen branches on every stage)
                if (!full) {
                    const bool out0 = j0 + pr * 32 + (lane & 15) >= cur.nb;
                    const bool out1 = j0 + pr * 32 + 16 + (lane & 15) >= cur.nb;
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            sc[0][rb][i] = out0 ? kNegInf : sc[0][rb][i];
                            sc[1][rb][i] = out1 ? kNegInf : sc[1][rb][i];
                        }
                }
                if (FIRST && pr == 0) {
                    // The item's first pair sets each row's reference from
                    // its own logits.  A lane whose first pair is masked has
                    // no valid position in the item at all (positions only
                    // grow), so a reference left at -FLT_MAX only ever meets
                    // masked logits: d = -inf, and it never moves.
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float v0 = sc[0][rb][i] * sl, v1 = sc[1][rb][i] * sl;
                            const float pv = fmaxf(v0, v1);
                            const float rn = pv > kNegInf ? pv + 16.f : -kFltMax;
                            mrun[h][rb][i] = rn;
                            zrun[h][rb][i] = __builtin_amdgcn_exp2f(v0 - rn) + __builtin_amdgcn_exp2f(v1 - rn);
                        }
                    continue;
                }
                // d = v - mrun for both logits, in place; a positive d passes
                // the reference
                bool pass_ref = false;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sc[0][rb][i] = __builtin_fmaf(sc[0][rb][i], sl, -mrun[h][rb][i]);
                        sc[1][rb][i] = __builtin_fmaf(sc[1][rb][i], sl, -mrun[h][rb][i]);
                        pass_ref |= (sc[0][rb][i] > 0.f) | (sc[1][rb][i] > 0.f);
                    }
                if (__ballot(pass_ref)) {   // rare after a row's first positions
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // the reference moves to the larger logit + 16
                            const float dm = fmaxf(sc[0][rb][i], sc[1][rb][i]);
                            const float up = dm > 0.f ? dm + 16.f : 0.f;
                            zrun[h][rb][i] *= __builtin_amdgcn_exp2f(-up);
                            mrun[h][rb][i] += up;
                            sc[0][rb][i] -= up;
                            sc[1][rb][i] -= up;
                        }
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        zrun[h][rb][i] += __builtin_amdgcn_exp2f(sc[0][rb][i]) + __builtin_amdgcn_exp2f(sc[1][rb][i]);
            }
            slot = (slot + 1) & (NSL - 1);
        };
        // The next item's page ids are requested before its Q fragments, so
        // the waits that follow cover them.  Steady case (a full ring on
        // entry and at least AHEAD + 2 stages): stages 0 and 1 each issue one
        // of this item's stages unconditionally, so at least 2 * NI requests
        // follow those loads before the counted waits of the last AHEAD
        // stages, which issue the next item's first stages and need its page
        // ids; the compiler can then see the loads complete without draining
        // the ring.  Other items settle the loads with one full wait.
        // (the loads sit on one path: loads in two branches became a
        // select of the two results, which waits for them)
        if (cur.nst > 0) stream_wait<AHEAD, GM::NI>(ci - 1);
        pgn = load_pg(nxt);
        stream_load_q<RB, NH>(a, nxt.b, nxt.l, nxt.h, qo, qn);
        if (cur.nst == 0) {
            wait_vmcnt<0>();
            top_up(-1);
        } else {
            const bool steady = ci == AHEAD && cur.nst >= AHEAD + 2;
            if (steady) {
                issue(cur, pg, ci++, ring[wave][islot]);
                islot = (islot + 1) & (NSL - 1);
                stage(0, std::true_type{});
                // at least one pass (cur.nst >= AHEAD + 2): written so, the
                // compiler sees two stages issued after the loads above on
                // every path and needs no wait of its own for them
                int s = 1;
                do {
                    wait_vmcnt<(AHEAD - 1) * GM::NI>();
                    issue(cur, pg, ci++, ring[wave][islot]);
                    islot = (islot + 1) & (NSL - 1);
                    stage(s, std::false_type{});
                } while (++s < cur.nst - AHEAD);
                // The last AHEAD stages each issue one of the next item's
                // first stages.  Unrolled: a loop here that reads the page ids
                // loaded outside it and issues DMA whose results it never
                // reads made the compiler drain every request before it.
#pragma unroll
                for (int t = 0; t < AHEAD; ++t) {
                    stream_wait<AHEAD, GM::NI>(AHEAD - 1 - t + min(t, nn));
                    if (t < nn) {
                        issue(nxt, pgn, t, ring[wave][islot]);
                        islot = (islot + 1) & (NSL - 1);
                    }
                    stage(cur.nst - AHEAD + t, std::false_type{});
                }
                ni = min(AHEAD, nn);
            } else {
                wait_vmcnt<0>();
                top_up(0);
                stage(0, std::true_type{});
                for (int s = 1; s < cur.nst; ++s) {
                    stream_wait<AHEAD, GM::NI>(ci - 1 - s + ni);
                    top_up(s);
                    stage(s, std::false_type{});
                }
            }
        }
        // combine the 16 token lanes of each row, then the four waves
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // a row with no valid position has a zero sum (its
                    // reference left at -FLT_MAX): reported as (-inf, 0)
                    const float mx = lane16_max(mrun[h][rb][i]);
                    const float mu = (mx == kNegInf) ? 0.f : mx;
                    const float z = lane16_sum(zrun[h][rb][i] * __builtin_amdgcn_exp2f(mrun[h][rb][i] - mu));
                    if ((lane & 15) == 0) {
                        const int r = rb * 16 + (lane >> 4) * 4 + i;
                        red[par][wave][h][r][0] = z > 0.f ? mx : kNegInf;
                        red[par][wave][h][r][1] = z;
                    }
                }
        lds_barrier();   // the next item's requests stay in flight
        if (threadIdx.x < NH * a.rows) {
            const int h = threadIdx.x / a.rows, r = threadIdx.x - h * a.rows;
            float rm[4], rz[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                rm[w] = lds_read_f32(&red[par][w][h][r][0]);
                rz[w] = lds_read_f32(&red[par][w][h][r][1]);
            }
            float mx = kNegInf;
#pragma unroll
            for (int w = 0; w < 4; ++w) mx = fmaxf(mx, rm[w]);
            const float mu = (mx == kNegInf) ? 0.f : mx;
            float z = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) z += rz[w] * __builtin_amdgcn_exp2f(rm[w] - mu);
            float *st = a.stat + ((((int64_t)cur.b * U + cur.l * 2 + cur.h + h) * a.rows + r) * nch + cur.c) * 2;
            st[0] = mx;
            st[1] = z;
        }
        par ^= 1;
        return ni;
    };
    int it = blockIdx.x;
    if (it >= items) return;
    bf16x8 qA[NH][RB][KK], qB[NH][RB][KK];
    Item cur = decode(it);
    stream_load_q<RB, NH>(a, cur.b, cur.l, cur.h, qo, qA);
    int pgA = load_pg(cur), pgB = 0;
    int ci = 0;   // stages of the current item already issued
    for (; ci < cur.nst && ci < AHEAD; ++ci) {
        issue(cur, pgA, ci, ring[wave][islot]);
        islot = (islot + 1) & (NSL - 1);
    }
    for (;;) {
        int nit = it + gridDim.x;
        Item nxt = decode(nit < items ? nit : it);
        ci = item(cur, nxt, nit < items, qA, qB, pgA, pgB, ci);
        if (nit >= items) break;
        it = nit;
        cur = nxt;
        nit = it + gridDim.x;
        nxt = decode(nit < items ? nit : it);
        ci = item(cur, nxt, nit < items, qB, qA, pgB, pgA, ci);
        if (nit >= items) break;
        it = nit;
        cur = nxt;
    }
}

// Layer groups of the streaming accumulation, chosen on the device from the
// actual chunk count (sum over sequences of ceil(n_b / 1024)): the count g <=
// cap (several groups: an even number of layers each) whose items (chunks x
// g x heads per item) take the fewest rounds of the persistent grid,
// weighted by the layers an item streams plus an eighth of a layer of fixed
// cost per item; ties to fewer groups.  The accumulation kernel and
// draft_part_sum evaluate it on the same arguments.
__device__ __forceinline__ int acc_layer_groups(int chunks, int nhi, int L, int cap, int grid) {
    int best = 1;
    long long best_cost = -1;
    for (int lg = 1; lg <= cap; ++lg) {
        int lpg = (L + lg - 1) / lg;
        if (lg > 1) lpg += lpg & 1;
        if ((L + lpg - 1) / lpg != lg) continue;   // not a count that even groups reach
        const long long items = (long long)chunks * lg * nhi;
        const long long cost = ((items + grid - 1) / grid) * (8LL * lpg + 1);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = lg;
        }
    }
    return best;
}

// Accumulation pass, streaming form.  Items (b, 1024-position chunk, layer
// group) walk round robin over the persistent groups (chunks wholly past n_b
// only write zeros); wave w owns positions w * 256 .. + 255 of the chunk and
// streams them layer after layer of its group, 8 stages per layer of full
// rows or 4 of half rows (stages past n_b are skipped).  With one layer
// group the item writes S_Draft; otherwise it writes its group's partial
// sum, added up by draft_part_sum.  A layer's page ids, Q fragments and row
// normalisers are requested by the previous layer's first stage,
// unconditionally and into the other of two named register sets.  Each
// stage adds sum_{head, row} exp2(logit - lse) for its positions to a
// wave-private LDS accumulator, in layer order, so S_Draft needs no atomics.
template <int RB, bool PAGED, bool HALF>
__global__ __launch_bounds__(256, 2) void draft_acc_stream(DraftScoreArgs a) {
    constexpr int KK = 2;
    constexpr int CHUNK = 1024;
    using GM = StreamGeom<RB, HALF>;
    constexpr int POS = GM::POS;
    constexpr int NH = GM::NH;                 // heads per item (HALF: one)
    constexpr int NHI = HALF ? 2 : 1;          // items per (b, chunk, layer group)
    constexpr int PER_WAVE = CHUNK / 4;
    constexpr int NSTAGE = PER_WAVE / POS;
    constexpr int NSL = GM::NSLOT;
    constexpr int AHEAD = NSL - 1;             // stages in flight beyond the one computed
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4][NSL][GM::STAGE];
    __shared__ float accs[4][PER_WAVE];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const KvView &k0 = a.kv[0];   // every draft layer has this geometry (checked on the host)
    const int N = k0.N_max;
    const int B = k0.B;
    // Items are (b, chunk, layer group) over the chunks that hold positions
    // below n_b only, numbered sequence by sequence (B <= kDraftStatMaxB).
    __shared__ int pref[kDraftStatMaxB + 1];
    for (int bb = threadIdx.x; bb < B; bb += blockDim.x) pref[bb + 1] = (sl_len(k0, bb) + CHUNK - 1) / CHUNK;
    __syncthreads();
    if (threadIdx.x == 0) {
        pref[0] = 0;
        for (int bb = 0; bb < B; ++bb) pref[bb + 1] += pref[bb];
    }
    __syncthreads();
    const int nchunks = __builtin_amdgcn_readfirstlane(pref[B]);   // uniform: the item loop is scalar
    const int LG = acc_layer_groups(nchunks, NHI, a.L_d, max(a.acc_groups, 1), gridDim.x);
    const int GT = LG * NHI;                   // partial groups: (layer group, head)
    const int items = nchunks * GT;
    if (GT == 1) {   // chunks wholly past n_b: S_Draft = 0 (with layer groups draft_part_sum writes them)
        for (int bb = 0; bb < B; ++bb) {
            const int j0 = (pref[bb + 1] - pref[bb]) * CHUNK;
            for (int j = j0 + blockIdx.x * 256 + (int)threadIdx.x; j < N; j += gridDim.x * 256)
                a.s_draft[(int64_t)bb * N + j] = 0.f;
        }
    }
    const int L = a.L_d;
    const int U = L * 2;
    // layers per group: ceil(L / LG) rounded up to even, so every group is
    // non-empty (with several groups L is even and so is every group; one
    // group takes all L layers, odd or even)
    const int lpg = ((L + LG - 1) / LG + 1) & ~1;
    // per-lane Q offsets, and normaliser offsets: rows rb*16 + (lane >> 4)*4
    // .. + 3 in one 16-byte load (the row count is a multiple of 4); rows past
    // the count read row 0's normalisers and are dropped where the terms are
    // summed (a select there, not on the loaded values, so no wait follows
    // the loads)
    uint32_t qo[RB], lo[RB];
    bool lok[RB];
    stream_qoff<RB>(a, lane, qo);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r4 = rb * 16 + (lane >> 4) * 4;
        lok[rb] = r4 < a.rows;
        lo[rb] = (uint32_t)(lok[rb] ? r4 : 0) * 4u;
    }
    auto load_lse = [&](int b, int l, int h0, f32x4 (&ls)[NH][RB]) {
        const __amdgpu_buffer_rsrc_t lr =
            stream_rsrc(a.lse + ((int64_t)b * U + l * 2) * a.rows, (uint32_t)(2 * a.rows * sizeof(float)));
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                ls[h][rb] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(lr, lo[rb], (h0 + h) * a.rows * 4, 0));
    };
    float *acc = accs[wave];
    int slot = 0, islot = 0;   // ring slots of the next stage to compute / to issue
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int bc = it / GT, gt = it - (it / GT) * GT;
        const int g = gt / NHI, h0 = gt - (gt / NHI) * NHI;   // layer group, head (HALF)
        int lo = 0, hi = B - 1;   // the b with pref[b] <= bc < pref[b + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pref[mid] <= bc) lo = mid;
            else hi = mid - 1;
        }
        // every item field is wave-uniform: readfirstlane makes that visible,
        // so the stage loops and the counted waits are scalar branches
        const int b = __builtin_amdgcn_readfirstlane(lo);
        const int c = __builtin_amdgcn_readfirstlane(bc - pref[lo]);
        const int l0 = g * lpg, l1 = min(L, l0 + lpg);
        const int nb = __builtin_amdgcn_readfirstlane(sl_len(k0, b));
        const int jw = c * CHUNK + __builtin_amdgcn_readfirstlane(wave) * PER_WAVE;
        const int left = nb - jw;
        const int nst = (left <= 0 || l0 >= l1) ? 0 : min(NSTAGE, (left + POS - 1) / POS);
#pragma unroll
        for (int i = 0; i < PER_WAVE / 64; ++i) acc[lane + 64 * i] = 0.f;
        if (nst > 0) {
            const int64_t seq0 = PAGED ? 0 : (int64_t)b * N * 256;
            // paged caches: the page ids of the wave's 256 positions (16
            // pages) in each layer, one per lane, loaded with the layer's Q
            auto load_pg = [&](int l) -> int { return PAGED ? stream_load_pg(a.kv[l], b, jw, PER_WAVE / 16, lane) : 0; };
            auto issue = [&](int l, const char *kl, int pgv, int s, uint8_t *stage) __attribute__((always_inline)) {
                if constexpr (PAGED) stream_issue_pg<POS, HALF>(kl, pgv, s, a.kv[l].num_pages, h0 * 128, lane, stage);
                else stream_issue<POS, HALF>(kl, jw + s * POS, N - 1, h0 * 128, lane, stage);
            };
            bf16x8 qA[NH][RB][KK], qB[NH][RB][KK];
            f32x4 lA[NH][RB], lB[NH][RB];
            int pA = 0, pB = 0;
            stream_load_q<RB, NH>(a, b, l0, h0, qo, qA);
            load_lse(b, l0, h0, lA);
            pA = load_pg(l0);
            int ci = 0;   // stages of the current layer already issued
            for (; ci < nst && ci < AHEAD; ++ci) {
                issue(l0, a.kv[l0].k + seq0, pA, ci, ring[wave][islot]);
                islot = (islot + 1) & (NSL - 1);
            }
            auto stage = [&](int s, const bf16x8 (&q)[NH][RB][KK], const f32x4 (&ls)[NH][RB]) {
                const uint32_t base = lds_addr(ring[wave][slot]);
#pragma unroll
                for (int s16 = 0; s16 < POS / 16; ++s16) {
                    float t = 0.f;
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        bf16x8 k[2];
                        stream_kfrag<HALF>(base, s16, h, lane, k);
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int kk = 0; kk < KK; ++kk)
                                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[h][rb][kk], k[kk], sc, 0, 0, 0);
                            float e = 0.f;
#pragma unroll
                            for (int i = 0; i < 4; ++i) e += __builtin_amdgcn_exp2f(sc[i] * a.scale_log2 - ls[h][rb][i]);
                            t += lok[rb] ? e : 0.f;
                        }
                    }
                    t = group4_sum(t);
                    if (lane < 16) acc[s * POS + s16 * 16 + lane] += t;
                }
                slot = (slot + 1) & (NSL - 1);
            };
            // One layer, `ci` of whose stages were issued before it began;
            // keeps AHEAD stages in flight, running on into the next layer of
            // the group, and returns how many of its stages it issued.
            auto layer = [&](int l, const bf16x8 (&q)[NH][RB][KK], const f32x4 (&ls)[NH][RB], const int &pg,
                             bf16x8 (&qn)[NH][RB][KK], f32x4 (&lsn)[NH][RB], int &pgn, int ci) -> int {
                ci = __builtin_amdgcn_readfirstlane(ci);
                // both layers' cache pointers from uniform indices (scalar
                // loads, outside the vector-load order)
                const int ln = (l + 1 < l1) ? l + 1 : l;
                const int nn = (l + 1 < l1) ? nst : 0;
                const char *kl = a.kv[l].k + seq0;
                const char *kn = a.kv[ln].k + seq0;
                int ni = 0;   // stages of the next layer issued
                auto top_up = [&](int s) __attribute__((always_inline)) {
                    while ((ci - 1 - s) + ni < AHEAD) {
                        const bool own = ci < nst;
                        if (!own && ni >= nn) break;
                        if (own) issue(l, kl, pg, ci, ring[wave][islot]);
                        else issue(ln, kn, pgn, ni, ring[wave][islot]);
                        ci += own ? 1 : 0;
                        ni += own ? 0 : 1;
                        islot = (islot + 1) & (NSL - 1);
                    }
                };
                // As in the statistics pass: the next layer's page ids ahead
                // of its Q and normalisers; in the steady case stages 0 and 1
                // issue this layer's stages unconditionally, so the counted
                // waits of the last AHEAD stages cover those loads.
                const bool steady = ci == AHEAD && nst >= AHEAD + 2;
                stream_wait<AHEAD, GM::NI>(ci - 1);
                pgn = load_pg(ln);
                stream_load_q<RB, NH>(a, b, ln, h0, qo, qn);
                load_lse(b, ln, h0, lsn);
                if (steady) {
                    issue(l, kl, pg, ci++, ring[wave][islot]);
                    islot = (islot + 1) & (NSL - 1);
                    stage(0, q, ls);
                    int s = 1;   // at least one pass (see the statistics pass)
                    do {
                        wait_vmcnt<(AHEAD - 1) * GM::NI>();
                        issue(l, kl, pg, ci++, ring[wave][islot]);
                        islot = (islot + 1) & (NSL - 1);
                        stage(s, q, ls);
                    } while (++s < nst - AHEAD);
                    // the last AHEAD stages, unrolled (see the statistics pass)
#pragma unroll
                    for (int t = 0; t < AHEAD; ++t) {
                        stream_wait<AHEAD, GM::NI>(AHEAD - 1 - t + min(t, nn));
                        if (t < nn) {
                            issue(ln, kn, pgn, t, ring[wave][islot]);
                            islot = (islot + 1) & (NSL - 1);
                        }
                        stage(nst - AHEAD + t, q, ls);
                    }
                    ni = min(AHEAD, nn);
                } else {
                    wait_vmcnt<0>();
                    top_up(0);
                    stage(0, q, ls);
                    for (int s = 1; s < nst; ++s) {
                        stream_wait<AHEAD, GM::NI>(ci - 1 - s + ni);
                        top_up(s);
                        stage(s, q, ls);
                    }
                }
                return ni;
            };
            // layer pairs with both calls unconditional (a conditional second
            // call made the compiler merge the two Q sets with selects, which
            // wait for the loads), then an odd last layer
            int l = l0;
            for (; l + 1 < l1; l += 2) {
                ci = layer(l, qA, lA, pA, qB, lB, pB, ci);
                ci = layer(l + 1, qB, lB, pB, qA, lA, pA, ci);
            }
            if (l < l1) layer(l, qA, lA, pA, qB, lB, pB, ci);
        }
        float *out = (GT == 1) ? a.s_draft + (int64_t)b * N : a.part + ((int64_t)gt * k0.B + b) * N;
#pragma unroll
        for (int i = 0; i < PER_WAVE / 64; ++i) {
            const int j = jw + lane + 64 * i;
            if (j < N) out[j] = (j < nb) ? acc[lane + 64 * i] : 0.f;
        }
    }
}

// --------------------------------------------------------------- host side
// Most layer groups the streaming accumulation may split a chunk's layers
// into (the device picks the count from the actual lengths, at most this):
// enough that items at full lengths would fill the persistent grid about 16
// times, at most L_d / 2 groups of two layers.  Depends on shapes only, so
// the workspace size needs no device.
int draft_acc_groups(int B, int N_max, int L_d) {
    if (L_d < 4 || L_d % 2 != 0) return 1;
    const long items = (long)B * ((N_max + 1023) / 1024);
    long lg = (16L * kStreamGroups + items - 1) / items;
    if (lg > L_d / 2) lg = L_d / 2;
    return lg <= 1 ? 1 : (int)lg;
}

// S_Draft = the partials (layer group, head) summed in group order; positions
// past n_b are 0 (the partials of chunks wholly past n_b are never written).
// With one partial the accumulation kernel has written S_Draft itself.
__global__ __launch_bounds__(256) void draft_part_sum(const float *part, int nhi, int cap, int L, int grid, int B,
                                                      int N, const int32_t *seq_lens, float *out, bool vec) {
    // the chunk count, with the lengths loaded in parallel (one load per
    // lane, then a block sum): a serial loop over B put B dependent loads in
    // front of the common case, one group, where nothing is left to do
    __shared__ int s_part[4];
    int c = 0;
    for (int bb = threadIdx.x; bb < B; bb += 256) c += (min(max(seq_lens[bb], 0), N) + 1023) / 1024;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = c;
    __syncthreads();
    const int chunks = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    const int groups = acc_layer_groups(chunks, nhi, L, cap, grid) * nhi;
    if (groups == 1) return;
    // row b = blockIdx.y; with vec, four positions per lane in 16-byte
    // accesses (N % 4 == 0, out and part 16-byte aligned: checked by the
    // launcher)
    const int64_t n = (int64_t)B * N;
    const int b = blockIdx.y;
    const int nb = __builtin_amdgcn_readfirstlane(min(max(seq_lens[b], 0), N));
    const float *pr = part + (int64_t)b * N;
    float *orow = out + (int64_t)b * N;
    if (vec) {
        for (int j = (blockIdx.x * 256 + threadIdx.x) * 4; j < N; j += gridDim.x * 1024) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (j < nb) {
                for (int g = 0; g < groups; ++g) {
                    const f32x4 u = *(const f32x4 *)(pr + (int64_t)g * n + j);
                    v[0] += u[0];
                    v[1] += u[1];
                    v[2] += u[2];
                    v[3] += u[3];
                }
#pragma unroll
                for (int e = 1; e < 4; ++e)   // a row that ends inside these four
                    if (j + e >= nb) v[e] = 0.f;
            }
            *(f32x4 *)(orow + j) = v;
        }
    } else {
        for (int j = blockIdx.x * 256 + threadIdx.x; j < N; j += gridDim.x * 256) {
            float v = 0.f;
            if (j < nb)
                for (int g = 0; g < groups; ++g) v += pr[(int64_t)g * n + j];
            orow[j] = v;
        }
    }
}

ScorePlan score_plan(int B, int N_max, int L_d, int H_d, int gamma, int S, int Hkv_d) {
    ScorePlan p{};
    p.nchunk = (N_max + CH - 1) / CH;
    (void)Hkv_d;
    const size_t drows = (size_t)L_d * gamma * H_d;   // rows over all draft (layer, KV head) units
    size_t off = 0;
    p.off_tlogit = off;
    off = align_up(off + (size_t)B * S * N_max * sizeof(float), 256);
    p.off_tstat = off;
    off = align_up(off + (size_t)B * S * p.nchunk * 2 * sizeof(float), 256);
    p.off_tlse = off;
    off = align_up(off + (size_t)B * S * sizeof(float), 256);
    p.off_dstat = off;
    off = align_up(off + (size_t)B * drows * p.nchunk * 2 * sizeof(float), 256);
    p.off_dlse = off;
    off = align_up(off + (size_t)B * drows * sizeof(float), 256);
    p.acc_groups = draft_acc_groups(B, N_max, L_d);
    p.off_dpart = off;
    // partial sums per (layer group, head): the one-head-per-item form
    // doubles the groups (its use depends on the draft's head geometry, which
    // the workspace query does not carry, so the space is always reserved)
    if (L_d >= 1) off = align_up(off + (size_t)2 * p.acc_groups * B * N_max * sizeof(float), 256);
    p.ws_bytes = off;
    return p;
}

// Supplied normalisers into the passes' layout.
static hipError_t import_draft_lse(const DraftScoreArgs &a, int B, hipStream_t s) {
    const int64_t n = (int64_t)B * a.L_d * a.gamma * a.H_d;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(draft_lse_import, dim3((unsigned)blocks), dim3(256), 0, s, a.lse_in, a.lse, n, a.L_d, a.gamma,
                       a.H_d, a.Hkv_d, a.G_d);
    return hipGetLastError();
}
// Row-normaliser query: the passes' normalisers out in the caller's layout.
static hipError_t export_draft_lse(const DraftScoreArgs &a, int B, hipStream_t s) {
    const int64_t n = (int64_t)B * a.L_d * a.gamma * a.H_d;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(draft_lse_export, dim3((unsigned)blocks), dim3(256), 0, s, a.lse, a.lse_out, n, a.L_d, a.gamma,
                       a.H_d, a.Hkv_d, a.G_d);
    return hipGetLastError();
}

template <bool F32, int D, int NV>
static hipError_t run_unit_stats(const ValuStatsParams<F32, D, NV> &p, int B, hipStream_t s) {
    dim3 grid(p.nchunk, p.ut.n_units, B);
    hipLaunchKernelGGL((unit_stats_valu<F32, D, NV>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <bool F32, int D>
static hipError_t target_impl(const TargetScoreArgs &a, hipStream_t s) {
    ValuStatsParams<F32, D, 8> p{};
    for (int i = 0; i < a.n_layers; ++i) p.kv[i] = a.kv[i];
    const KvView &k0 = a.kv[0];
    // one unit per (layer, kv head) with at most 8 rows, rows kept in order
    UnitTable &ut = p.ut;
    ut.n_units = 0;
    for (int r = 0; r < a.S;) {
        int n = 1;
        while (r + n < a.S && n < 8 && a.row_layer[r + n] == a.row_layer[r] && a.row_kvh[r + n] == a.row_kvh[r]) ++n;
        ut.view[ut.n_units] = a.row_layer[r];
        ut.kvh[ut.n_units] = a.row_kvh[r];
        ut.row0[ut.n_units] = r;
        ut.nrow[ut.n_units] = n;
        ++ut.n_units;
        r += n;
    }
    p.q = (const char *)a.q_hist;
    p.q_bstride = (int64_t)a.S * D;
    for (int r = 0; r < a.S; ++r) p.qoff[r] = r * D;
    p.total_rows = a.S;
    p.scale_log2 = a.scale_log2;
    p.stat = a.stat;
    p.logit = a.logit;
    p.nchunk = a.nchunk;
    p.N_max = k0.N_max;
    // whole-row form: bf16, head_dim 128, one layer, every KV head exactly one unit
    bool rows_form = !F32 && D == 128 && a.n_layers == 1 && ut.n_units == k0.Hkv && k0.Hkv <= 16 &&
                     (k0.Hkv & (k0.Hkv - 1)) == 0;
    int unit_of_head[16];
    for (int h = 0; h < 16; ++h) unit_of_head[h] = -1;
    for (int u = 0; rows_form && u < ut.n_units; ++u) {
        if (unit_of_head[ut.kvh[u]] >= 0) rows_form = false;
        else unit_of_head[ut.kvh[u]] = u;
    }
    hipError_t e;
    if (rows_form) {
        RowStatsParams q{};
        q.kv = k0;
        q.q = (const char *)a.q_hist;
        q.S = a.S;
        for (int h = 0; h < 16; ++h) q.unit_of_head[h] = unit_of_head[h] < 0 ? 0 : unit_of_head[h];
        for (int u = 0; u < ut.n_units; ++u) {
            q.row0[u] = ut.row0[u];
            q.nrow[u] = ut.nrow[u];
        }
        q.scale_log2 = a.scale_log2;
        q.stat = a.stat;
        q.logit = a.logit;
        q.nchunk = a.nchunk;
        q.N_max = k0.N_max;
        int nr_max = 1;
        for (int u = 0; u < ut.n_units; ++u) nr_max = ut.nrow[u] > nr_max ? ut.nrow[u] : nr_max;
        if (nr_max > 4) {
            // matrix-core form: split the KV heads over work-groups until the
            // chunks fill the chip four times over (or one head per group)
            const int Hkv = k0.Hkv;
            int hsplit = 1;
            while (hsplit < Hkv && (int64_t)a.nchunk * k0.B * hsplit < 4 * 256) hsplit *= 2;
            while (Hkv / hsplit > 8) hsplit *= 2;   // at most 8 heads (64 KiB of logits) per group
            const int HPG = Hkv / hsplit;
            const int wph = HPG >= 4 ? 1 : 4 / HPG;
            const dim3 grid(a.nchunk, k0.B, hsplit);
            const size_t lds = (size_t)HPG * 8 * kRowsMfmaLdsStride * sizeof(float);
            if (HPG >= 8) hipLaunchKernelGGL(unit_stats_rows_mfma<2>, grid, dim3(256), lds, s, q, HPG, wph);
            else hipLaunchKernelGGL(unit_stats_rows_mfma<1>, grid, dim3(256), lds, s, q, HPG, wph);
        } else {
            const dim3 grid(a.nchunk, k0.B);
            const size_t lds = (size_t)a.S * CH * sizeof(float);
            if (nr_max == 1) hipLaunchKernelGGL(unit_stats_rows<1>, grid, dim3(256), lds, s, q);
            else if (nr_max == 2) hipLaunchKernelGGL(unit_stats_rows<2>, grid, dim3(256), lds, s, q);
            else hipLaunchKernelGGL(unit_stats_rows<4>, grid, dim3(256), lds, s, q);
        }
        e = hipGetLastError();
    } else {
        e = run_unit_stats(p, k0.B, s);
    }
    if (e != hipSuccess) return e;
    float *lse = a.lse;
    hipLaunchKernelGGL(rows_lse, dim3((k0.B * a.S + 3) / 4), dim3(256), 0, s, a.stat, lse, k0.B * a.S, a.nchunk,
                       k0.seq_lens, a.S, CH, k0.N_max);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.rows_out) {
        if (k0.N_max % 4 == 0 && ((uintptr_t)a.rows_out | (uintptr_t)a.logit) % 16 == 0)
            hipLaunchKernelGGL(target_rows_finalize<true>, dim3((k0.N_max / 4 + 255) / 256, k0.B, a.S), dim3(256), 0,
                               s, a.logit, lse, a.rows_out, k0.seq_lens, k0.B, a.S, k0.N_max);
        else
            hipLaunchKernelGGL(target_rows_finalize<false>, dim3((k0.N_max + 255) / 256, k0.B, a.S), dim3(256), 0, s,
                               a.logit, lse, a.rows_out, k0.seq_lens, k0.B, a.S, k0.N_max);
    } else {
        if (k0.N_max % 4 == 0 && ((uintptr_t)a.s_target | (uintptr_t)a.logit) % 16 == 0)
            hipLaunchKernelGGL(target_finalize<true>, dim3((k0.N_max / 4 + 255) / 256, k0.B), dim3(256), 0, s,
                               a.logit, lse, a.s_target, k0.seq_lens, a.S, k0.N_max);
        else
            hipLaunchKernelGGL(target_finalize<false>, dim3((k0.N_max + 255) / 256, k0.B), dim3(256), 0, s, a.logit,
                               lse, a.s_target, k0.seq_lens, a.S, k0.N_max);
    }
    return hipGetLastError();
}

hipError_t launch_target_score(const TargetScoreArgs &a, hipStream_t s) {
    const KvView &k0 = a.kv[0];
    if (k0.f32) {
        switch (k0.D) {
            case 32: return target_impl<true, 32>(a, s);
            case 64: return target_impl<true, 64>(a, s);
            case 128: return target_impl<true, 128>(a, s);
        }
    } else {
        switch (k0.D) {
            case 32: return target_impl<false, 32>(a, s);
            case 64: return target_impl<false, 64>(a, s);
            case 128: return target_impl<false, 128>(a, s);
        }
    }
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t draft_f32_impl(const DraftScoreArgs &a, hipStream_t s) {
    // float32 drafts are small (tests, tiny configs): at most 8 layers, and
    // units of <= 8 rows.
    const KvView &k0 = a.kv[0];
    if (a.L_d > 8) return hipErrorInvalidValue;
    ValuStatsParams<true, D, 8> p{};
    for (int i = 0; i < a.L_d; ++i) p.kv[i] = a.kv[i];
    UnitTable &ut = p.ut;
    ut.n_units = 0;
    int row = 0;
    for (int l = 0; l < a.L_d; ++l)
        for (int c = 0; c < a.Hkv_d; ++c)
            for (int r0 = 0; r0 < a.rows; r0 += 8) {
                if (ut.n_units >= kMaxScoreRows) return hipErrorInvalidValue;
                const int n = (a.rows - r0 < 8) ? a.rows - r0 : 8;
                ut.view[ut.n_units] = l;
                ut.kvh[ut.n_units] = c;
                ut.row0[ut.n_units] = row;
                ut.nrow[ut.n_units] = n;
                for (int i = 0; i < n; ++i) {
                    const int r = r0 + i, gs = r / a.G_d, hh = r - (r / a.G_d) * a.G_d;
                    if (row + i >= kMaxScoreQoff) return hipErrorInvalidValue;
                    p.qoff[row + i] = ((l * a.gamma + gs) * a.H_d + c * a.G_d + hh) * D;
                }
                row += n;
                ++ut.n_units;
            }
    p.q = (const char *)a.q_draft;
    p.q_bstride = (int64_t)a.L_d * a.gamma * a.H_d * D;
    p.total_rows = row;
    p.scale_log2 = a.scale_log2;
    p.stat = a.stat;
    p.logit = nullptr;
    p.nchunk = a.nchunk;
    p.N_max = k0.N_max;
    hipError_t e;
    if (a.lse_in) {
        if ((e = import_draft_lse(a, k0.B, s)) != hipSuccess) return e;
    } else {
        if ((e = run_unit_stats(p, k0.B, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(rows_lse, dim3((k0.B * row + 3) / 4), dim3(256), 0, s, a.stat, a.lse, k0.B * row, a.nchunk,
                           k0.seq_lens, row, CH, k0.N_max);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.lse_out) return export_draft_lse(a, k0.B, s);
    DraftValuAccParams<D, 8> q{};
    for (int i = 0; i < a.L_d; ++i) q.kv[i] = a.kv[i];
    q.ut = ut;
    q.q = p.q;
    q.q_bstride = p.q_bstride;
    for (int i = 0; i < row; ++i) q.qoff[i] = p.qoff[i];
    q.total_rows = row;
    q.scale_log2 = a.scale_log2;
    q.lse = a.lse;
    q.out = a.s_draft;
    q.N_max = k0.N_max;
    hipLaunchKernelGGL((draft_acc_valu<D, 8>), dim3(a.nchunk, k0.B), dim3(256), 0, s, q);
    return hipGetLastError();
}

// Streaming passes: two 64-wide draft KV heads and a row count that is a
// multiple of four; contiguous or paged; HALF (three or four row blocks):
// one KV head per item.
template <int RB, bool PAGED, bool HALF>
static hipError_t draft_stream_impl(const DraftScoreArgs &a, hipStream_t s) {
    const KvView &k0 = a.kv[0];
    DraftScoreArgs b = a;
    constexpr int NHI = HALF ? 2 : 1;
    constexpr int GROUPS = StreamGeom<RB, HALF>::GROUPS;
    // Statistics items of twice the positions halve the per-item combine
    // when there are still at least two per persistent group (contiguous
    // caches: a paged wave span holds one page id per lane).  Measured at
    // c4: 504 -> 490 us; at c2 (B = 4, 16k) the larger items underfill the
    // chip, so the rule keeps 4096 there.
    constexpr int CH2 = 2 * kDraftStatChunk;
    const bool big = !PAGED && (long)k0.B * a.L_d * NHI * ((k0.N_max + CH2 - 1) / CH2) >= 2L * GROUPS;
    const int chunk = big ? CH2 : kDraftStatChunk;
    b.nchunk = (k0.N_max + chunk - 1) / chunk;
    const int stat_items = k0.B * a.L_d * NHI * b.nchunk;
    hipError_t e;
    if (a.lse_in) {
        if ((e = import_draft_lse(a, k0.B, s)) != hipSuccess) return e;
    } else {
        const dim3 grid(stat_items < GROUPS ? stat_items : GROUPS);
        if constexpr (!PAGED) {
            if (big) hipLaunchKernelGGL((draft_stats_stream<RB, PAGED, HALF, CH2>), grid, dim3(256), 0, s, b);
            else hipLaunchKernelGGL((draft_stats_stream<RB, PAGED, HALF>), grid, dim3(256), 0, s, b);
        } else {
            hipLaunchKernelGGL((draft_stats_stream<RB, PAGED, HALF>), grid, dim3(256), 0, s, b);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int nrows = k0.B * a.L_d * 2 * a.rows;
        hipLaunchKernelGGL(rows_lse, dim3((nrows + 3) / 4), dim3(256), 0, s, b.stat, b.lse, nrows, b.nchunk,
                           k0.seq_lens, a.L_d * 2 * a.rows, chunk, k0.N_max);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.lse_out) return export_draft_lse(a, k0.B, s);
    const int cap = a.acc_groups > 1 ? a.acc_groups : 1;   // the device picks <= cap layer groups
    b.acc_groups = cap;
    const long acc_items = (long)k0.B * ((k0.N_max + 1023) / 1024) * cap * NHI;   // at full lengths
    const int grid = acc_items < GROUPS ? (int)acc_items : GROUPS;
    hipLaunchKernelGGL((draft_acc_stream<RB, PAGED, HALF>), dim3(grid), dim3(256), 0, s, b);
    if ((e = hipGetLastError()) != hipSuccess || cap * NHI == 1) return e;
    const bool vec = k0.N_max % 4 == 0 && (uintptr_t)a.s_draft % 16 == 0 && (uintptr_t)a.part % 16 == 0;
    const int per_block = vec ? 1024 : 256;   // positions of a row per work-group and round
    const int bx = std::min((k0.N_max + per_block - 1) / per_block, 256);
    hipLaunchKernelGGL(draft_part_sum, dim3((unsigned)bx, (unsigned)k0.B), dim3(256), 0, s, a.part, NHI, cap, a.L_d,
                       grid, k0.B, k0.N_max, k0.seq_lens, a.s_draft, vec);
    return hipGetLastError();
}

template <int D, int RB>
static hipError_t draft_bf16_impl(const DraftScoreArgs &a, hipStream_t s) {
    const KvView &k0 = a.kv[0];
    if constexpr (D == 64) {
        constexpr bool HALF = RB >= 3;
        if (a.Hkv_d == 2 && a.rows % 4 == 0)
            return k0.page_size == 0 ? draft_stream_impl<RB, false, HALF>(a, s) : draft_stream_impl<RB, true, HALF>(a, s);
    }
    const int U = a.L_d * a.Hkv_d;
    DraftScoreArgs b = a;
    b.nchunk = (k0.N_max + kDraftStatChunk - 1) / kDraftStatChunk;
    const int stat_items = k0.B * U * b.nchunk;
    hipError_t e;
    if (a.lse_in) {
        if ((e = import_draft_lse(a, k0.B, s)) != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((draft_stats_mfma<D, RB>), dim3(stat_items < kScoreGroups ? stat_items : kScoreGroups),
                           dim3(256), 0, s, b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int nrows = k0.B * U * a.rows;
        hipLaunchKernelGGL(rows_lse, dim3((nrows + 3) / 4), dim3(256), 0, s, b.stat, b.lse, nrows, b.nchunk,
                           k0.seq_lens, U * a.rows, kDraftStatChunk, k0.N_max);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.lse_out) return export_draft_lse(a, k0.B, s);
    const int acc_items = k0.B * ((k0.N_max + kDraftAccChunk - 1) / kDraftAccChunk);
    const dim3 grid(acc_items < kScoreGroups ? acc_items : kScoreGroups);
    if (k0.page_size != 0) hipLaunchKernelGGL((draft_acc_mfma<D, RB, true>), grid, dim3(256), 0, s, b);
    else hipLaunchKernelGGL((draft_acc_mfma<D, RB, false>), grid, dim3(256), 0, s, b);
    return hipGetLastError();
}

// Window attention A of Eq. (1) through the draft machinery: statistics pass,
// row normalisers, then the per-step accumulation (a.gamma <= 4 steps).
template <int D, int RB>
static hipError_t window_bf16_impl(const DraftScoreArgs &a, hipStream_t s) {
    const KvView &k0 = a.kv[0];
    const int U = a.L_d * a.Hkv_d;
    DraftScoreArgs b = a;
    b.nchunk = (k0.N_max + kDraftStatChunk - 1) / kDraftStatChunk;
    const int stat_items = k0.B * U * b.nchunk;
    hipLaunchKernelGGL((draft_stats_mfma<D, RB>), dim3(stat_items < kScoreGroups ? stat_items : kScoreGroups),
                       dim3(256), 0, s, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nrows = k0.B * U * a.rows;
    hipLaunchKernelGGL(rows_lse, dim3((nrows + 3) / 4), dim3(256), 0, s, b.stat, b.lse, nrows, b.nchunk, k0.seq_lens,
                       U * a.rows, kDraftStatChunk, k0.N_max);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int acc_items = k0.B * ((k0.N_max + kDraftAccChunk - 1) / kDraftAccChunk);
    const dim3 grid(acc_items < kScoreGroups ? acc_items : kScoreGroups);
    const bool sa = a.G_d % 4 == 0;
    if (k0.page_size != 0) {
        if (sa) hipLaunchKernelGGL((draft_acc_mfma<D, RB, true, 4, true>), grid, dim3(256), 0, s, b);
        else hipLaunchKernelGGL((draft_acc_mfma<D, RB, true, 4, false>), grid, dim3(256), 0, s, b);
    } else {
        if (sa) hipLaunchKernelGGL((draft_acc_mfma<D, RB, false, 4, true>), grid, dim3(256), 0, s, b);
        else hipLaunchKernelGGL((draft_acc_mfma<D, RB, false, 4, false>), grid, dim3(256), 0, s, b);
    }
    return hipGetLastError();
}

hipError_t launch_window_steps(const DraftScoreArgs &a, hipStream_t s) {
    const int RB = (a.rows + 15) / 16;
    if (a.kv[0].f32 || a.gamma > 4 || RB > 4) return hipErrorInvalidValue;
#define DUSTIN_WINDOW_CASE(DD)                                 \
    switch (RB) {                                              \
        case 1: return window_bf16_impl<DD, 1>(a, s);          \
        case 2: return window_bf16_impl<DD, 2>(a, s);          \
        case 3: return window_bf16_impl<DD, 3>(a, s);          \
        case 4: return window_bf16_impl<DD, 4>(a, s);          \
    }                                                          \
    return hipErrorInvalidValue;
    switch (a.kv[0].D) {
        case 32: DUSTIN_WINDOW_CASE(32)
        case 64: DUSTIN_WINDOW_CASE(64)
        case 128: DUSTIN_WINDOW_CASE(128)
    }
#undef DUSTIN_WINDOW_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_draft_score(const DraftScoreArgs &a, hipStream_t s) {
    const KvView &k0 = a.kv[0];
    if (k0.f32) {
        switch (k0.D) {
            case 32: return draft_f32_impl<32>(a, s);
            case 64: return draft_f32_impl<64>(a, s);
            case 128: return draft_f32_impl<128>(a, s);
        }
        return hipErrorInvalidValue;
    }
    const int RB = (a.rows + 15) / 16;
#define DUSTIN_DRAFT_CASE(DD)                                  \
    switch (RB) {                                              \
        case 1: return draft_bf16_impl<DD, 1>(a, s);           \
        case 2: return draft_bf16_impl<DD, 2>(a, s);           \
        case 3: return draft_bf16_impl<DD, 3>(a, s);           \
        case 4: return draft_bf16_impl<DD, 4>(a, s);           \
    }                                                          \
    return hipErrorInvalidValue;
    switch (k0.D) {
        case 32: DUSTIN_DRAFT_CASE(32)
        case 64: DUSTIN_DRAFT_CASE(64)
        case 128: DUSTIN_DRAFT_CASE(128)
    }
#undef DUSTIN_DRAFT_CASE
    return hipErrorInvalidValue;
}

}  // namespace dustin
