// Verification-set selection (Dustin blog section 2.3) for gfx950: one global
// index set per sequence, shared by every layer and head (section 2.2).
//
//   tier 0  P = attention sinks [0, n_sink) and recent window [n - n_window, n)
//   tier 1  D = the m' positions outside P with the largest S_Draft
//   tier 2  T = the positions outside P u D with the largest S_Target,
//           filling the budget k
// Ties go to the lower position.  The result is written in ascending order.
//
// One 1024-lane work-group per sequence.  Each TopK is a most-significant-
// digit radix select on the float bit patterns (scores are non-negative, so
// the unsigned order of the bits is the numeric order) that finds the k-th
// largest key T and how many keys equal to T are needed; every key above T
// then goes in, plus the lowest positions among the keys equal to T.
// Sequences up to 131072 positions keep their selections in registers
// (topk_il_kernel, below); longer ones keep per-position tier flags in the
// workspace (topk_kernel: three passes of 11/11/10-bit digits with the
// histogram in LDS; position j is always handled by lane j mod 1024, so the
// flags need no synchronisation beyond the block barriers).

#include "common.h"
#include "internal.h"

namespace dustin {

constexpr int TKT = 1024;            // lanes per work-group
constexpr int TKW = TKT / 64;        // waves

struct TopkShared {
    unsigned hist[2048];
    int wave_tot[TKW];
    int digit;
    int above;
};

// Exclusive prefix count of `pred` over the work-group in lane order, plus
// the total.  Two barriers.
__device__ __forceinline__ int block_scan(bool pred, int &total, TopkShared &sh) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const unsigned long long m = __ballot(pred);
    const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) sh.wave_tot[wave] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < TKW; ++w) {
        const int c = sh.wave_tot[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + in_wave;
}

// Select the K largest candidate scores (flag == 0) of one sequence and set
// their flag to `tag`.  Requires 1 <= K <= number of candidates.
__device__ void select_top(const float *sc, uint8_t *flag, int n, int K, int ncand, uint8_t tag, TopkShared &sh) {
    const int tid = threadIdx.x;
    if (K >= ncand) {
        for (int j = tid; j < n; j += TKT)
            if (flag[j] == 0) flag[j] = tag;
        __syncthreads();
        return;
    }
    uint32_t prefix = 0, mask = 0;
    int remaining = K;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int sh_ = shifts[pass], wd = widths[pass];
        const uint32_t dmask = (1u << wd) - 1u;
        const int nbins = 1 << wd;
        for (int i = tid; i < nbins; i += TKT) sh.hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += TKT) {
            if (flag[j] != 0) continue;
            const uint32_t key = __float_as_uint(sc[j]);
            if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> sh_) & dmask], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            const int lane = tid;
            const int per = nbins / 64;
            int local = 0;
            for (int i = 0; i < per; ++i) local += (int)sh.hist[lane * per + i];
            // above[lane] = sum of local over lanes > lane
            int incl = local;   // inclusive suffix sum
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_down(incl, o, 64);
                if (lane + o < 64) incl += v;
            }
            const int above = incl - local;
            if (above < remaining && remaining <= incl) {
                int acc = above;
                for (int i = per - 1; i >= 0; --i) {
                    const int d = lane * per + i;
                    const int c = (int)sh.hist[d];
                    if (acc + c >= remaining) {
                        sh.digit = d;
                        sh.above = acc;
                        break;
                    }
                    acc += c;
                }
            }
        }
        __syncthreads();
        remaining -= sh.above;
        prefix |= (uint32_t)sh.digit << sh_;
        mask |= dmask << sh_;
        __syncthreads();
    }
    const uint32_t thr = prefix;
    const int need = remaining;   // keys equal to thr still to take
    int taken = 0;
    for (int base = 0; base < n; base += TKT) {
        const int j = base + tid;
        bool tie = false;
        if (j < n && flag[j] == 0) {
            const uint32_t key = __float_as_uint(sc[j]);
            if (key > thr) flag[j] = tag;
            tie = (key == thr);
        }
        int tot;
        const int rank = taken + block_scan(tie, tot, sh);
        if (tie && rank < need) flag[j] = tag;
        taken += tot;
    }
    __syncthreads();
}

__global__ __launch_bounds__(TKT) void topk_kernel(TopkArgs a) {
    __shared__ TopkShared sh;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int n = min(max(a.seq_lens[a.len_mod ? b % a.len_mod : b], 0), a.N_max);
    uint8_t *flag = a.flag + (int64_t)b * a.N_max;
    const int se = min(a.n_sink, n);
    const int wb = max(0, n - a.n_window);
    const int np = se + (n - max(wb, se));
    const int budget = a.k - np;
    const int rest = n - np;
    int m_eff = a.s_draft ? (a.s_target ? a.m : budget) : 0;
    m_eff = max(0, min(m_eff, min(budget, rest)));
    const int t_cnt = max(0, min(budget - m_eff, rest - m_eff));

    for (int j = tid; j < n; j += TKT) flag[j] = (j < se || j >= wb) ? 1 : 0;
    __syncthreads();
    if (m_eff > 0) select_top(a.s_draft + (int64_t)(a.d_mod ? b % a.d_mod : b) * a.N_max, flag, n, m_eff, rest, 2, sh);
    if (t_cnt > 0) select_top(a.s_target + (int64_t)(a.t_mod ? b % a.t_mod : b) * a.N_max, flag, n, t_cnt, rest - m_eff, 3, sh);

    int32_t *idx = a.idx + (int64_t)b * a.k;
    int8_t *tier = a.tier ? a.tier + (int64_t)b * a.k : nullptr;
    int written = 0;
    for (int base = 0; base < n; base += TKT) {
        const int j = base + tid;
        const uint8_t f = (j < n) ? flag[j] : 0;
        int tot;
        const int pos = written + block_scan(f != 0, tot, sh);
        if (f != 0 && pos < a.k) {
            idx[pos] = j;
            if (tier) tier[pos] = (int8_t)(f - 1);
        }
        written += tot;
    }
    const int cnt = min(written, a.k);
    for (int p = cnt + tid; p < a.k; p += TKT) {
        idx[p] = -1;
        if (tier) tier[p] = -1;
    }
    if (tid == 0) a.count[b] = cnt;
}

// ----------------------------------------------------------------------------
// Register-resident variant (n <= 32 * MW * 1024, MW <= 4; longer sequences
// use the kernel above).  Lane t owns the positions j = 1024 i + t of the
// rows i = 0 .. 32 MW - 1, so every key load of a wave reads 64 consecutive
// floats.  The lane's draft / target selections are bit masks in registers
// (bit b of word w = row 32 w + b).  Position order is row-major, so the
// order-dependent steps (ties at the threshold, the ascending compaction)
// take one wave ballot per row and one block-wide prefix over the
// (row, wave) counts.
//
// Each radix pass histograms the candidate keys inside the current window
// [lo, hi] of the bit-pattern order with the digit (key - lo) >> s, s chosen
// so that the window spans at most 2048 bins.  The first window is the
// candidates' own [min, max], so the bins follow where the keys actually lie
// (with the top bits of the float pattern as the digit, the keys of a
// narrow value range share a few bins and the histogram atomics serialise).
// Every pass narrows the window to the bin holding the K-th largest key,
// which leaves fewer than 2^s patterns, so the search ends after at most
// three passes with a window of one key value, or earlier when the bin's
// keys are exactly the ones still needed.

constexpr int kIlMaxRows = 128;     // rows per lane at MW = 4
constexpr int kIlHistCopies = 4;    // waves w and w + 4k share histogram copy w % 4

struct alignas(16) TopkIlShared {
    unsigned hist[kIlHistCopies][2048];
    int rowcnt[kIlMaxRows * TKW];   // per (row, wave) counts, then their exclusive prefixes
    int wave_tot[TKW];
    uint32_t wmin[TKW], wmax[TKW];
    int digit, above, inbin;
};

// Exclusive prefix sum of v over the work-group in lane order, plus the total.
__device__ __forceinline__ int block_prefix(int v, int &total, int *wave_tot) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < TKW; ++w) {
        const int c = wave_tot[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// In-place exclusive prefix of cnt[0 .. ne) in index order (ne <= 2 * TKT);
// returns the total.  Ends with a barrier, so the prefixes are visible.
__device__ __forceinline__ int block_scan_array(int *cnt, int ne, int *wave_tot) {
    const int e = 2 * threadIdx.x;
    const int a0 = (e < ne) ? cnt[e] : 0, a1 = (e + 1 < ne) ? cnt[e + 1] : 0;
    int total;
    const int before = block_prefix(a0 + a1, total, wave_tot);
    if (e < ne) cnt[e] = before;
    if (e + 1 < ne) cnt[e + 1] = before + a0;
    __syncthreads();
    return total;
}

// Keys of rows 32 w .. 32 w + 31 of this lane through a buffer resource
// bounded at n keys: positions >= n read 0 (the candidate masks never
// include them) with no per-lane branch, and the row offset is an immediate
// (scalar) operand, so no per-row address is kept in registers.
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t rs, int w, uint32_t (&kw)[32]) {
    const uint32_t voff = threadIdx.x * 4u;
#pragma unroll
    for (int bit = 0; bit < 32; ++bit)
        kw[bit] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, voff, (w * 32 + bit) * TKT * 4, 0);
}

// Number of this lane's rows whose position 1024 i + t lies below p.
__device__ __forceinline__ int rows_below(int p) {
    const int t = threadIdx.x;
    return p > t ? (p - t + TKT - 1) / TKT : 0;
}

// Bits of word w for the rows r with r0 <= r < r1.
__device__ __forceinline__ uint32_t row_bits(int w, int r0, int r1) {
    const int a = min(max(r0 - 32 * w, 0), 32), b = min(max(r1 - 32 * w, 0), 32);
    return (uint32_t)(((1ull << b) - 1ull) & ~((1ull << a) - 1ull));
}

// Rank the lane's bits of `m` in row-major position order over the
// work-group (count per (row, wave), block prefix, then the ballot offset),
// calling f(w, bit, rank) for each set bit.  Rows from `nrows` on must hold
// no set bit.  Every lane must call it.
// The 16 waves of the work-group share one CU, so the per-row loops are kept
// free of branches and LDS round trips: a word's 32 row counts are gathered
// into lanes 0..31 (a select per row) and stored with one instruction, and after
// the scan the 32 prefixes come back with one LDS read and readlane.
template <int MW, class F>
__device__ __forceinline__ int rank_rows(const uint32_t (&m)[MW], int nrows, TopkIlShared &sh, F &&f) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    (void)nrows;   // rows from nrows on hold no set bit: they count zero
#pragma unroll
    for (int w = 0; w < MW; ++w) {
        int cnt = 0;   // lane r < 32: set bits of row w * 32 + r in this wave
#pragma unroll
        for (int bit = 0; bit < 32; ++bit) {
            // every lane takes part in the ballot; only lane `bit` keeps its count
            const int pc = (int)__popcll(__ballot((m[w] >> bit) & 1u));
            cnt = (lane == bit) ? pc : cnt;
        }
        if (lane < 32) sh.rowcnt[(w * 32 + lane) * TKW + wave] = cnt;
    }
    __syncthreads();
    const int total = block_scan_array(sh.rowcnt, 32 * MW * TKW, sh.wave_tot);
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
        if (__ballot(m[w] != 0u) == 0ull) continue;   // no lane of the wave has a set bit in this word
        const int pre = sh.rowcnt[(w * 32 + (lane & 31)) * TKW + wave];   // lane r: prefix of row w * 32 + r
#pragma unroll
        for (int bit = 0; bit < 32; ++bit) {
            const bool mine = (m[w] >> bit) & 1u;
            const unsigned long long bal = __ballot(mine);
            if (mine) f(w, bit, __builtin_amdgcn_readlane(pre, bit) + __popcll(bal & lt));
        }
    }
    __syncthreads();   // rowcnt may be reused
    return total;
}

// Select the K largest candidate keys (the bits of cm), setting their bits
// in `sel`; ties at the threshold go to the lower positions.  Requires
// 1 <= K; K >= ncand takes every candidate.
template <int MW>
__device__ void select_top_il(const float *sc, int n, const uint32_t (&cm)[MW], uint32_t (&sel)[MW], int K,
                              int ncand, TopkIlShared &sh) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (K >= ncand) {
#pragma unroll
        for (int w = 0; w < MW; ++w) sel[w] = cm[w];
        return;
    }
    constexpr bool CACHE = MW == 1;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(sc), (short)0, n * 4, 0x00020000);
    uint32_t kc[32];
    if constexpr (CACHE) load_rows(rs, 0, kc);
    auto each_word = [&](auto &&f) {
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            if (w * 32 * TKT >= n) break;   // uniform: no position of this word is below n
            if constexpr (CACHE) {
                f(w, kc);
            } else {
                // the keys are read again by every pass: keep the compiler
                // from hoisting the reads of all words (32 MW registers) out
                asm volatile("" ::: "memory");
                uint32_t kw[32];
                load_rows(rs, w, kw);
                f(w, kw);
            }
        }
    };
    // first window: [min, max] of the candidate keys
    uint32_t lo = 0xffffffffu, hi = 0u;
    each_word([&](int w, const uint32_t (&kw)[32]) {
#pragma unroll
        for (int bit = 0; bit < 32; ++bit)
            if ((cm[w] >> bit) & 1u) {
                lo = min(lo, kw[bit]);
                hi = max(hi, kw[bit]);
            }
    });
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    }
    if (lane == 0) {
        sh.wmin[wave] = lo;
        sh.wmax[wave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < TKW; ++w) {
        lo = min(lo, sh.wmin[w]);
        hi = max(hi, sh.wmax[w]);
    }
    int remaining = K;    // keys still to take from the window
    bool exact = false;   // every key of the window is taken
    unsigned *hc = sh.hist[wave % kIlHistCopies];
    // The histogram is zero on entry (cleared at the kernel's start, and
    // every pass's scan zeroes the counters it reads), so a pass needs no
    // clear of its own; the barrier after the scan orders those zeroes
    // before the next pass's atomics.
    for (int pass = 0; pass < 4; ++pass) {   // the window shrinks to one value within three passes
        const uint32_t r = hi - lo;
        const int bl = r ? 32 - __clz((int)r) : 0;
        const int s = max(0, bl - 11);
        each_word([&](int w, const uint32_t (&kw)[32]) {
#pragma unroll
            for (int bit = 0; bit < 32; ++bit) {
                const uint32_t key = kw[bit];
                if (((cm[w] >> bit) & 1u) && key >= lo && key <= hi) atomicAdd(&hc[(key - lo) >> s], 1u);
            }
        });
        __syncthreads();
        {   // bin holding the remaining-th largest key, from the top: wave v
            // owns bins 128 v .. 128 v + 127, lane l the pair 128 v + 2 l, + 1
            const int b0 = wave * 128 + 2 * lane;
            int c0 = 0, c1 = 0;
#pragma unroll
            for (int c = 0; c < kIlHistCopies; ++c) {
                const uint2 h = *(const uint2 *)&sh.hist[c][b0];
                c0 += (int)h.x;
                c1 += (int)h.y;
            }
#pragma unroll
            for (int c = 0; c < kIlHistCopies; ++c) *(uint2 *)&sh.hist[c][b0] = uint2{0u, 0u};
            // every lane read the previous pass's result before the
            // histogram barrier above, so it can be reset here
            if (tid == 0) {
                sh.digit = 0;
                sh.above = 0;
                sh.inbin = 0;
            }
            const int local = c0 + c1;
            int incl = local;   // inclusive suffix sum over lanes >= lane
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_down(incl, o, 64);
                if (lane + o < 64) incl += v;
            }
            if (lane == 0) sh.wave_tot[wave] = incl;   // the wave's bin total
            __syncthreads();
            int above_w = 0;   // keys in the bins of the waves above this one
#pragma unroll
            for (int v = 0; v < TKW; ++v) above_w += (v > wave) ? sh.wave_tot[v] : 0;
            const int above = above_w + incl - local;
            if (above < remaining && remaining <= above + local) {
                const bool hi_bin = above + c1 >= remaining;
                sh.digit = b0 + (hi_bin ? 1 : 0);
                sh.above = hi_bin ? above : above + c1;
                sh.inbin = hi_bin ? c1 : c0;
            }
        }
        __syncthreads();
        remaining -= sh.above;
        const int inbin = sh.inbin;
        lo += (uint32_t)sh.digit << s;
        hi = min(hi, lo + ((1u << s) - 1u));
        if (remaining == inbin) {
            exact = true;
            break;
        }
        if (s == 0) break;
    }
    // keys above the window all go in; of the window, either every key
    // (exact) or, the window being one value, the lowest positions holding it
    uint32_t tie[MW];
    int ties = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) sel[w] = tie[w] = 0;
    each_word([&](int w, const uint32_t (&kw)[32]) {
        uint32_t m = 0, t = 0;
#pragma unroll
        for (int bit = 0; bit < 32; ++bit) {
            const bool c = (cm[w] >> bit) & 1u;
            m |= (uint32_t)(c && (kw[bit] > hi || (exact && kw[bit] >= lo))) << bit;
            t |= (uint32_t)(c && !exact && kw[bit] == lo) << bit;
        }
        sel[w] = m;
        tie[w] = t;
        ties += __popc(t);
    });
    if (exact) return;
    int total;
    (void)block_prefix(ties, total, sh.wave_tot);
    if (total <= remaining) {
#pragma unroll
        for (int w = 0; w < MW; ++w) sel[w] |= tie[w];
        return;
    }
    const int need = remaining;
    rank_rows<MW>(tie, (n + TKT - 1) / TKT, sh, [&](int w, int bit, int rank) {
        if (rank < need) sel[w] |= 1u << bit;
    });
}

template <int MW>
__global__ __launch_bounds__(TKT) void topk_il_kernel(TopkArgs a) {
    __shared__ TopkIlShared sh;
    const int b = blockIdx.x, tid = threadIdx.x;
    // the radix passes expect a zero histogram (each pass leaves it zero);
    // the barrier inside the first selection orders this before any atomic
    for (int i = tid; i < kIlHistCopies * 2048; i += TKT) (&sh.hist[0][0])[i] = 0u;
    if (tid == 0) {
        sh.digit = 0;
        sh.above = 0;
        sh.inbin = 0;
    }
    const int n = min(max(a.seq_lens[a.len_mod ? b % a.len_mod : b], 0), a.N_max);
    const int se = min(a.n_sink, n);
    const int wb = max(0, n - a.n_window);
    const int np = se + (n - max(wb, se));
    const int budget = a.k - np;
    const int rest = n - np;
    int m_eff = a.s_draft ? (a.s_target ? a.m : budget) : 0;
    m_eff = max(0, min(m_eff, min(budget, rest)));
    const int t_cnt = max(0, min(budget - m_eff, rest - m_eff));

    uint32_t cm[MW], pm[MW], dsel[MW], tsel[MW];   // candidates, protected, draft tier, target tier
    {
        const int r_n = rows_below(n), r_se = rows_below(se), r_wb = rows_below(wb);
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            const uint32_t valid = row_bits(w, 0, r_n);
            const uint32_t prot = row_bits(w, 0, r_se) | row_bits(w, r_wb, r_n);
            cm[w] = valid & ~prot;
            pm[w] = valid & prot;
            dsel[w] = tsel[w] = 0;
        }
    }
    if (m_eff > 0)
        select_top_il<MW>(a.s_draft + (int64_t)(a.d_mod ? b % a.d_mod : b) * a.N_max, n, cm, dsel, m_eff, rest, sh);
#pragma unroll
    for (int w = 0; w < MW; ++w) cm[w] &= ~dsel[w];
    if (t_cnt > 0)
        select_top_il<MW>(a.s_target + (int64_t)(a.t_mod ? b % a.t_mod : b) * a.N_max, n, cm, tsel, t_cnt,
                          rest - m_eff, sh);

    // ascending compaction: rank every kept position in row-major order
    uint32_t keep[MW];
#pragma unroll
    for (int w = 0; w < MW; ++w) keep[w] = pm[w] | dsel[w] | tsel[w];
    int32_t *idx = a.idx + (int64_t)b * a.k;
    int8_t *tier = a.tier ? a.tier + (int64_t)b * a.k : nullptr;
    const int written = rank_rows<MW>(keep, (n + TKT - 1) / TKT, sh, [&](int w, int bit, int pos) {
        if (pos < a.k) {
            idx[pos] = (w * 32 + bit) * TKT + tid;
            if (tier) tier[pos] = (int8_t)(((pm[w] >> bit) & 1u) ? 0 : (((dsel[w] >> bit) & 1u) ? 1 : 2));
        }
    });
    const int cnt = min(written, a.k);
    for (int p = cnt + tid; p < a.k; p += TKT) {
        idx[p] = -1;
        if (tier) tier[p] = -1;
    }
    if (tid == 0) a.count[b] = cnt;
}

// ----------------------------------------------------------------------------
// Chunked variant for long rows (kMwMinN <= N_max <= kMwMaxN): a sequence is
// cut into chunks of 4096 positions, one 256-lane work-group per chunk, so a
// long row's radix passes run on many CUs instead of one.  Lane t of chunk c
// owns the positions j = 4096 c + 256 i + t, rows i = 0 .. 15 (each key load
// of a wave reads 64 consecutive floats); position order inside a chunk is
// row-major, as in the register-resident kernel.
//
// The passes are separate launches (the order of the stream is the only
// synchronisation between them):
//   mw_begin     tier flags of the sinks and the recent window; per-chunk
//                [min, max] of the first selection's candidate keys
//   mw_pass x3   histogram of the candidate keys inside the current window
//                (2048 bins, digit (key - lo) >> s, as in the register-
//                resident kernel), written per chunk; the work-group that
//                arrives last sums the chunks' histograms, finds the bin of
//                the remaining-th largest key and narrows the window
//   mw_mark      keys above the window, or, when the window ended as one
//                value, the lowest positions holding it: the ties before a
//                chunk are the other chunks' counts in the last pass's bin;
//                then the next selection's per-chunk [min, max] or the
//                chunk's kept count
//   mw_compact   ascending positions, each chunk at the prefix of the kept
//                counts of the chunks before it
// Three passes always suffice: the first window spans < 2^32 patterns, so
// s <= 21, then s <= 10, then s = 0.  A pass whose search has ended returns
// at once.  Data read across work-groups of one launch (the histograms, the
// arrival counter) goes through device-coherent accesses.

constexpr int MWT = 256;                   // lanes per chunk work-group
constexpr int MWW = MWT / 64;              // waves
constexpr int MWR = 16;                    // positions per lane
constexpr int MWC = MWT * MWR;             // positions per chunk
constexpr int kMwBins = 2048;
// A chunk's histogram in global memory holds 16-bit counts (a chunk has
// MWC = 4096 positions), two bins per word, so the work-group that sums the
// chunks' histograms reads a lane's eight bins of one chunk with one 16-byte
// load and keeps every chunk's load in flight at once.
constexpr int kMwHistWords = kMwBins / 2;
static_assert(MWC < 65536, "16-bit chunk histogram counts");
constexpr int kMwMaxChunks = 64;
constexpr int kMwMinN = 32768 + 1;         // shorter rows: the register-resident kernel
constexpr int kMwMaxN = kMwMaxChunks * MWC;

struct MwState {
    uint32_t lo, hi;       // the window of key patterns still open
    int32_t remaining;     // keys still to take from the window
    int32_t exact;         // every key of the window is taken
    int32_t fin;           // the search has ended
    int32_t tie_bin;       // last pass's bin of the threshold value (ranking of ties)
    int32_t pad[2];
};

struct MwPtrs {
    uint32_t *flag;        // [B][C][MWT] 2-bit tier codes of the lane's 16 rows
    uint32_t *mm;          // [B][C][2] per-chunk min / max candidate pattern
    int32_t *kept;         // [B][C] kept positions per chunk
    uint32_t *hist;        // [B][C][kMwHistWords] per-chunk histogram of the current pass (16-bit bins)
    MwState *state;        // [B][2] per selection (0 draft, 1 target)
    int32_t *ctr;          // [B] arrival counter of the current pass
    int C;
};

struct MwLayout {
    size_t off_flag, off_mm, off_kept, off_hist, off_state, off_ctr, bytes;
    int C;
};

MwLayout mw_layout(int B, int N_max) {
    MwLayout L{};
    L.C = (N_max + MWC - 1) / MWC;
    const size_t BC = (size_t)B * L.C;
    size_t off = 0;
    L.off_flag = off;
    off = align_up(off + BC * MWT * 4, 256);
    L.off_mm = off;
    off = align_up(off + BC * 2 * 4, 256);
    L.off_kept = off;
    off = align_up(off + BC * 4, 256);
    L.off_hist = off;
    off = align_up(off + BC * kMwBins * 4, 256);
    L.off_state = off;
    off = align_up(off + (size_t)B * 2 * sizeof(MwState), 256);
    L.off_ctr = off;
    off = align_up(off + (size_t)B * 4, 256);
    L.bytes = off;
    return L;
}

// Tier sizes of sequence b (the same arithmetic as the kernels above).
struct MwTiers {
    int n, se, wb, rest, m_eff, t_cnt;
};
__device__ __forceinline__ MwTiers mw_tiers(const TopkArgs &a, int b) {
    MwTiers T;
    T.n = min(max(a.seq_lens[a.len_mod ? b % a.len_mod : b], 0), a.N_max);
    T.se = min(a.n_sink, T.n);
    T.wb = max(0, T.n - a.n_window);
    const int np = T.se + (T.n - max(T.wb, T.se));
    const int budget = a.k - np;
    T.rest = T.n - np;
    int m_eff = a.s_draft ? (a.s_target ? a.m : budget) : 0;
    T.m_eff = max(0, min(m_eff, min(budget, T.rest)));
    T.t_cnt = max(0, min(budget - T.m_eff, T.rest - T.m_eff));
    return T;
}
// Selection `sel` of sequence b: its score row, K and candidate count.
__device__ __forceinline__ const float *mw_row(const TopkArgs &a, int b, int sel) {
    return sel == 0 ? a.s_draft + (int64_t)(a.d_mod ? b % a.d_mod : b) * a.N_max
                    : a.s_target + (int64_t)(a.t_mod ? b % a.t_mod : b) * a.N_max;
}
__device__ __forceinline__ void mw_sel(const MwTiers &T, int sel, int &K, int &ncand) {
    K = sel == 0 ? T.m_eff : T.t_cnt;
    ncand = sel == 0 ? T.rest : T.rest - T.m_eff;
}

__device__ __forceinline__ uint32_t ld_coherent_u32(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent_u32(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct MwShared {
    unsigned hist[kMwBins];
    int wave_tot[MWW];
    uint32_t red_lo[MWW], red_hi[MWW];
    int rowcnt[MWR * MWW];
    int flag;
    uint32_t b_lo, b_hi;
    int b_rem, b_digit, b_above, b_inbin;
};

// Block-wide min and max (every lane gets them).
__device__ __forceinline__ void mw_minmax(uint32_t &lo, uint32_t &hi, MwShared &sh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    }
    if (lane == 0) {
        sh.red_lo[wave] = lo;
        sh.red_hi[wave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < MWW; ++w) {
        lo = min(lo, sh.red_lo[w]);
        hi = max(hi, sh.red_hi[w]);
    }
    __syncthreads();
}

// Block-wide exclusive prefix of v in lane order, plus the total.
__device__ __forceinline__ int mw_prefix(int v, int &total, MwShared &sh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    if (lane == 63) sh.wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < MWW; ++w) {
        const int c = sh.wave_tot[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// Rank the lane's set bits of `m` (bit i = row i) in the chunk's position
// order, calling f(i, rank) for each; returns the chunk's total.
template <class F>
__device__ __forceinline__ int mw_rank(uint32_t m, MwShared &sh, F &&f) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < MWR; ++i) {
        const unsigned long long bal = __ballot((m >> i) & 1u);
        if (lane == 0) sh.rowcnt[i * MWW + wave] = __popcll(bal);
    }
    __syncthreads();
    // exclusive prefix over the 64 (row, wave) counts in (row, wave) order
    int total = 0;
    if (wave == 0) {
        const int v = sh.rowcnt[lane];
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o, 64);
            if (lane >= o) incl += u;
        }
        sh.rowcnt[lane] = incl - v;
        if (lane == 63) sh.wave_tot[0] = incl;
    }
    __syncthreads();
    total = sh.wave_tot[0];
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < MWR; ++i) {
        const bool mine = (m >> i) & 1u;
        const unsigned long long bal = __ballot(mine);
        if (mine) f(i, sh.rowcnt[i * MWW + wave] + __popcll(bal & lt));
    }
    __syncthreads();
    return total;
}

// Sum over the lanes of the block (every lane gets it).
__device__ __forceinline__ int mw_sum(int v, MwShared &sh) {
    int total;
    (void)mw_prefix(v, total, sh);
    return total;
}

// The lane's 16 keys of score row `row` (nullptr: none), requested for every
// position below N_max whether or not it turns out to be a candidate, so the
// loads wait for no other result (the length, the tier codes, the window).
__device__ __forceinline__ void mw_load_keys(const float *row, int j0, int N_max, uint32_t (&key)[MWR]) {
#pragma unroll
    for (int i = 0; i < MWR; ++i) {
        const int j = j0 + i * MWT;
        key[i] = (row != nullptr && j < N_max) ? __float_as_uint(row[j]) : 0u;
    }
}

// Candidate keys of rows `cand` of this lane: per-chunk min and max, stored
// by lane 0.
__device__ __forceinline__ void mw_store_minmax(const uint32_t (&key)[MWR], uint32_t cand, MwShared &sh,
                                                uint32_t *mm) {
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < MWR; ++i)
        if ((cand >> i) & 1u) {
            lo = min(lo, key[i]);
            hi = max(hi, key[i]);
        }
    mw_minmax(lo, hi, sh);
    if (threadIdx.x == 0) {
        st_coherent_u32(mm, lo);
        st_coherent_u32(mm + 1, hi);
    }
}

// Rows of this lane whose position is below n.
__device__ __forceinline__ uint32_t mw_valid(int j0, int n) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < MWR; ++i) v |= (uint32_t)(j0 + i * MWT < n) << i;
    return v;
}
// Rows whose 2-bit tier code is 0 (not kept so far).
__device__ __forceinline__ uint32_t mw_free(uint32_t fw) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < MWR; ++i) v |= (uint32_t)(((fw >> (2 * i)) & 3u) == 0u) << i;
    return v;
}

__global__ __launch_bounds__(MWT) void mw_begin(TopkArgs a, MwPtrs p) {
    __shared__ MwShared sh;
    const int b = blockIdx.x / p.C, c = blockIdx.x - (blockIdx.x / p.C) * p.C, t = threadIdx.x;
    const int j0 = c * MWC + t;
    const int sel = a.s_draft ? 0 : 1;   // the first selection of the call
    uint32_t key[MWR];                   // requested together with the length
    mw_load_keys((a.s_draft || a.s_target) ? mw_row(a, b, sel) : nullptr, j0, a.N_max, key);
    const MwTiers T = mw_tiers(a, b);
    const uint32_t valid = mw_valid(j0, T.n);
    uint32_t fw = 0, prot = 0;
#pragma unroll
    for (int i = 0; i < MWR; ++i) {
        const int j = j0 + i * MWT;
        prot |= (uint32_t)(((valid >> i) & 1u) && (j < T.se || j >= T.wb)) << i;
    }
#pragma unroll
    for (int i = 0; i < MWR; ++i) fw |= ((prot >> i) & 1u) << (2 * i);
    p.flag[((size_t)b * p.C + c) * MWT + t] = fw;
    int K, ncand;
    mw_sel(T, sel, K, ncand);
    if (K > 0 && K < ncand) mw_store_minmax(key, valid & ~prot, sh, p.mm + ((size_t)b * p.C + c) * 2);
    if (c == 0 && t == 0) __hip_atomic_store(&p.ctr[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int SEL>
__global__ __launch_bounds__(MWT) void mw_pass(TopkArgs a, MwPtrs p, int pass) {
    __shared__ MwShared sh;
    const int b = blockIdx.x / p.C, c = blockIdx.x - (blockIdx.x / p.C) * p.C, t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    // Every load of the pass is requested before any result is used: the
    // keys, the tier codes, the chunks' [min, max] or the window, and the
    // length (one round trip instead of a chain of them).
    const int j0 = c * MWC + t;
    uint32_t key[MWR];
    mw_load_keys(mw_row(a, b, SEL), j0, a.N_max, key);
    const uint32_t fw = p.flag[((size_t)b * p.C + c) * MWT + t];
    MwState *st = p.state + (size_t)b * 2 + SEL;
    uint32_t lo = 0xffffffffu, hi = 0u;
    if (pass == 0) {
        if (t < p.C) {
            lo = ld_coherent_u32(p.mm + ((size_t)b * p.C + t) * 2);
            hi = ld_coherent_u32(p.mm + ((size_t)b * p.C + t) * 2 + 1);
        }
    } else if (t == 0) {
        sh.flag = (int)ld_coherent_u32((const uint32_t *)&st->fin);
        sh.b_lo = ld_coherent_u32(&st->lo);
        sh.b_hi = ld_coherent_u32(&st->hi);
        sh.b_rem = (int)ld_coherent_u32((const uint32_t *)&st->remaining);
    }
    const MwTiers T = mw_tiers(a, b);
    int K, ncand;
    mw_sel(T, SEL, K, ncand);
    if (K <= 0 || K >= ncand) return;   // the same for every chunk of the sequence
    int remaining;
    if (pass == 0) {
        mw_minmax(lo, hi, sh);
        remaining = K;
    } else {
        __syncthreads();
        if (sh.flag) return;
        lo = sh.b_lo;
        hi = sh.b_hi;
        remaining = sh.b_rem;
    }
    const uint32_t r = hi - lo;
    const int bl = r ? 32 - __clz((int)r) : 0;
    const int s = max(0, bl - 11);
    for (int i = t; i < kMwBins; i += MWT) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t cand = mw_valid(j0, T.n) & mw_free(fw);
#pragma unroll
    for (int i = 0; i < MWR; ++i)
        if ((cand >> i) & 1u)
            if (key[i] >= lo && key[i] <= hi) atomicAdd(&sh.hist[(key[i] - lo) >> s], 1u);
    __syncthreads();
    // this chunk's histogram, written through: lane t packs bins 8t .. 8t + 7
    // into one 16-byte store
    uint32_t *hrow = p.hist + ((size_t)b * p.C + c) * kMwHistWords;
    const __amdgpu_buffer_rsrc_t hr = coherent_rsrc(hrow, kMwHistWords * 4);
    {
        const u32x4 lo4 = *(const u32x4 *)&sh.hist[8 * t], hi4 = *(const u32x4 *)&sh.hist[8 * t + 4];
        const u32x4 pk = {lo4[0] | (lo4[1] << 16), lo4[2] | (lo4[3] << 16), hi4[0] | (hi4[1] << 16),
                          hi4[2] | (hi4[3] << 16)};
        __builtin_amdgcn_raw_buffer_store_b128(pk, hr, (uint32_t)(16 * t), 0, kCachePolicySc1);
    }
    wait_all_mem();
    __syncthreads();
    if (t == 0) sh.flag = __hip_atomic_fetch_add(&p.ctr[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.C - 1;
    __syncthreads();
    if (!sh.flag) return;
    // last to arrive: sum the chunks' histograms (lane t: bins 8t .. 8t + 7)
    uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const __amdgpu_buffer_rsrc_t hall =
        coherent_rsrc(p.hist + (size_t)b * p.C * kMwHistWords, (uint32_t)(p.C * kMwHistWords * 4));
    // 32 chunks' loads in flight before any is added, one round for up to
    // 131072 positions (loads past the last chunk fall outside the resource
    // and read 0)
    for (int c0 = 0; c0 < p.C; c0 += 32) {
        u32x4 u[32];
#pragma unroll
        for (int q = 0; q < 32; ++q)
            u[q] = __builtin_amdgcn_raw_buffer_load_b128(hall, (uint32_t)(((c0 + q) * kMwHistWords + 4 * t) * 4), 0,
                                                         kCachePolicySc1);
#pragma unroll
        for (int q = 0; q < 32; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[2 * e] += u[q][e] & 0xffffu;
                h[2 * e + 1] += u[q][e] >> 16;
            }
    }
    int local = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) local += (int)h[q];
    // keys in the bins of the lanes above this one (higher bins = larger keys)
    int incl = local;   // inclusive suffix sum within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(incl, o, 64);
        if (lane + o < 64) incl += v;
    }
    if (lane == 0) sh.wave_tot[wave] = incl;
    __syncthreads();
    int above = incl - local;
#pragma unroll
    for (int w = 0; w < MWW; ++w) above += (w > wave) ? sh.wave_tot[w] : 0;
    if (above < remaining && remaining <= above + local) {
        int acc = above;
#pragma unroll
        for (int q = 7; q >= 0; --q) {
            const int cq = (int)h[q];
            if (acc < remaining && remaining <= acc + cq) {
                sh.b_digit = 8 * t + q;
                sh.b_above = acc;
                sh.b_inbin = cq;
            }
            acc += cq;
        }
    }
    __syncthreads();
    if (t == 0) {
        const int rem = remaining - sh.b_above;
        const uint32_t nlo = lo + ((uint32_t)sh.b_digit << s);
        const uint32_t nhi = min(hi, nlo + ((1u << s) - 1u));
        const int exact = rem == sh.b_inbin;
        st_coherent_u32(&st->lo, nlo);
        st_coherent_u32(&st->hi, nhi);
        st_coherent_u32((uint32_t *)&st->remaining, (uint32_t)rem);
        st_coherent_u32((uint32_t *)&st->exact, (uint32_t)exact);
        st_coherent_u32((uint32_t *)&st->fin, (uint32_t)(exact || s == 0));
        st_coherent_u32((uint32_t *)&st->tie_bin, (uint32_t)sh.b_digit);
        __hip_atomic_store(&p.ctr[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Mark the selection SEL in the chunk's tier codes; then either the per-chunk
// [min, max] of the target candidates (next_mm) or the chunk's kept count.
template <int SEL>
__global__ __launch_bounds__(MWT) void mw_mark(TopkArgs a, MwPtrs p, int next_mm, int count) {
    __shared__ MwShared sh;
    const int b = blockIdx.x / p.C, c = blockIdx.x - (blockIdx.x / p.C) * p.C, t = threadIdx.x;
    // requests first (keys of this selection and, for the next one's
    // [min, max], of the target row; tier codes; the window), then the length
    const int j0 = c * MWC + t;
    uint32_t key[MWR], tkey[MWR];
    mw_load_keys(mw_row(a, b, SEL), j0, a.N_max, key);
    mw_load_keys(next_mm ? mw_row(a, b, 1) : nullptr, j0, a.N_max, tkey);
    uint32_t *fwp = p.flag + ((size_t)b * p.C + c) * MWT + t;
    uint32_t fw = *fwp;
    const MwState *st = p.state + (size_t)b * 2 + SEL;
    if (t == 0) {
        sh.b_lo = ld_coherent_u32(&st->lo);
        sh.b_hi = ld_coherent_u32(&st->hi);
        sh.b_rem = (int)ld_coherent_u32((const uint32_t *)&st->remaining);
        sh.b_above = (int)ld_coherent_u32((const uint32_t *)&st->exact);
        sh.b_digit = (int)ld_coherent_u32((const uint32_t *)&st->tie_bin);
    }
    const MwTiers T = mw_tiers(a, b);
    int K, ncand;
    mw_sel(T, SEL, K, ncand);
    const uint32_t valid = mw_valid(j0, T.n);
    const uint32_t cand = valid & mw_free(fw);
    uint32_t sel = 0;
    if (K > 0 && K >= ncand) {
        sel = cand;
    } else if (K > 0) {
        __syncthreads();
        const uint32_t lo = sh.b_lo, hi = sh.b_hi;
        const int exact = sh.b_above, tie_bin = sh.b_digit, remaining = sh.b_rem;
        uint32_t tie = 0;
#pragma unroll
        for (int i = 0; i < MWR; ++i)
            if ((cand >> i) & 1u) {
                sel |= (uint32_t)(key[i] > hi || (exact && key[i] >= lo)) << i;
                tie |= (uint32_t)(!exact && key[i] == lo) << i;
            }
        if (!exact) {
            // ties in the chunks before this one: their counts in the last
            // pass's bin of the threshold value
            int before = 0;
            if (t < c) {
                const uint32_t w2 =
                    ld_coherent_u32(p.hist + ((size_t)b * p.C + t) * kMwHistWords + (tie_bin >> 1));
                before = (int)((tie_bin & 1) ? (w2 >> 16) : (w2 & 0xffffu));
            }
            before = mw_sum(before, sh);
            const int need = remaining - before;
            mw_rank(tie, sh, [&](int i, int rank) {
                if (rank < need) sel |= 1u << i;
            });
        }
    }
    const uint32_t code = SEL == 0 ? 2u : 3u;
#pragma unroll
    for (int i = 0; i < MWR; ++i) fw |= (((sel >> i) & 1u) * code) << (2 * i);
    *fwp = fw;
    if (next_mm) {
        int Kt, nct;
        mw_sel(T, 1, Kt, nct);
        if (Kt > 0 && Kt < nct) mw_store_minmax(tkey, valid & mw_free(fw), sh, p.mm + ((size_t)b * p.C + c) * 2);
    }
    if (count) {
        const int kept = mw_sum(__popc(valid & ~mw_free(fw)), sh);
        if (t == 0) st_coherent_u32((uint32_t *)&p.kept[(size_t)b * p.C + c], (uint32_t)kept);
    }
}

__global__ __launch_bounds__(MWT) void mw_compact(TopkArgs a, MwPtrs p) {
    __shared__ MwShared sh;
    const int b = blockIdx.x / p.C, c = blockIdx.x - (blockIdx.x / p.C) * p.C, t = threadIdx.x;
    const MwTiers T = mw_tiers(a, b);
    const int j0 = c * MWC + t;
    const uint32_t valid = mw_valid(j0, T.n);
    const uint32_t fw = p.flag[((size_t)b * p.C + c) * MWT + t];
    const uint32_t keep = valid & ~mw_free(fw);
    const int kc = (t < p.C) ? (int)ld_coherent_u32((const uint32_t *)&p.kept[(size_t)b * p.C + t]) : 0;
    int total;
    const int ex = mw_prefix(kc, total, sh);   // lane c holds the kept positions before chunk c
    if (t == c) sh.b_above = ex;
    __syncthreads();
    const int before = sh.b_above;
    int32_t *idx = a.idx + (int64_t)b * a.k;
    int8_t *tier = a.tier ? a.tier + (int64_t)b * a.k : nullptr;
    mw_rank(keep, sh, [&](int i, int rank) {
        const int pos = before + rank;
        if (pos < a.k) {
            idx[pos] = j0 + i * MWT;
            if (tier) tier[pos] = (int8_t)(((fw >> (2 * i)) & 3u) - 1u);
        }
    });
    const int cnt = min(total, a.k);
    for (int q = cnt + c * MWT + t; q < a.k; q += p.C * MWT) {
        idx[q] = -1;
        if (tier) tier[q] = -1;
    }
    if (c == 0 && t == 0) a.count[b] = cnt;
}

static hipError_t launch_topk_mw(const TopkArgs &a, hipStream_t s) {
    const MwLayout L = mw_layout(a.B, a.N_max);
    char *ws = (char *)a.flag;
    MwPtrs p{};
    p.flag = (uint32_t *)(ws + L.off_flag);
    p.mm = (uint32_t *)(ws + L.off_mm);
    p.kept = (int32_t *)(ws + L.off_kept);
    p.hist = (uint32_t *)(ws + L.off_hist);
    p.state = (MwState *)(ws + L.off_state);
    p.ctr = (int32_t *)(ws + L.off_ctr);
    p.C = L.C;
    const dim3 grid((unsigned)(a.B * L.C)), block(MWT);
    hipLaunchKernelGGL(mw_begin, grid, block, 0, s, a, p);
    if (a.s_draft) {
        for (int pass = 0; pass < 3; ++pass) hipLaunchKernelGGL(mw_pass<0>, grid, block, 0, s, a, p, pass);
        hipLaunchKernelGGL(mw_mark<0>, grid, block, 0, s, a, p, a.s_target ? 1 : 0, a.s_target ? 0 : 1);
    }
    if (a.s_target) {
        for (int pass = 0; pass < 3; ++pass) hipLaunchKernelGGL(mw_pass<1>, grid, block, 0, s, a, p, pass);
        hipLaunchKernelGGL(mw_mark<1>, grid, block, 0, s, a, p, 0, 1);
    }
    hipLaunchKernelGGL(mw_compact, grid, block, 0, s, a, p);
    return hipGetLastError();
}

TopkPlan topk_plan(int B, int N_max, int k) {
    (void)k;
    TopkPlan p{};
    p.off_flag = 0;
    if (N_max < kMwMinN) p.ws_bytes = 256;                          // register-resident: no workspace
    else if (N_max <= kMwMaxN) p.ws_bytes = mw_layout(B, N_max).bytes;
    else p.ws_bytes = align_up((size_t)B * N_max, 256);
    return p;
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    const int P = (a.N_max + TKT - 1) / TKT;   // positions per lane
    if (a.N_max >= kMwMinN && a.N_max <= kMwMaxN) return launch_topk_mw(a, s);
    if (P <= 32) hipLaunchKernelGGL(topk_il_kernel<1>, dim3(a.B), dim3(TKT), 0, s, a);
    else hipLaunchKernelGGL(topk_kernel, dim3(a.B), dim3(TKT), 0, s, a);
    return hipGetLastError();
}

}  // namespace dustin
