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
template <int MW, class F>
__device__ __forceinline__ int rank_rows(const uint32_t (&m)[MW], int nrows, TopkIlShared &sh, F &&f) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int w = 0; w < MW; ++w)
#pragma unroll 1
        for (int bit = 0; bit < 32; ++bit) {
            const int row = w * 32 + bit;
            const unsigned long long bal = (row < nrows) ? __ballot((m[w] >> bit) & 1u) : 0ull;
            if (lane == 0) sh.rowcnt[row * TKW + wave] = __popcll(bal);
        }
    __syncthreads();
    const int total = block_scan_array(sh.rowcnt, 32 * MW * TKW, sh.wave_tot);
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
        if (w * 32 >= nrows) break;
#pragma unroll 1
        for (int bit = 0; bit < 32; ++bit) {
            const bool mine = (m[w] >> bit) & 1u;
            const unsigned long long bal = __ballot(mine);
            if (mine) f(w, bit, sh.rowcnt[(w * 32 + bit) * TKW + wave] + __popcll(bal & lt));
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
    unsigned *hflat = &sh.hist[0][0];
    unsigned *hc = sh.hist[wave % kIlHistCopies];
    for (int pass = 0; pass < 4; ++pass) {   // the window shrinks to one value within three passes
        const uint32_t r = hi - lo;
        const int bl = r ? 32 - __clz((int)r) : 0;
        const int s = max(0, bl - 11);
        for (int i = tid; i < kIlHistCopies * 2048; i += TKT) hflat[i] = 0;
        if (tid == 0) {
            sh.digit = 0;
            sh.above = 0;
            sh.inbin = 0;
        }
        __syncthreads();
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
        __syncthreads();   // every lane has read digit / above / inbin before the next pass resets them
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

TopkPlan topk_plan(int B, int N_max, int k) {
    (void)k;
    TopkPlan p{};
    p.off_flag = 0;
    p.ws_bytes = align_up((size_t)B * N_max, 256);
    return p;
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    const int P = (a.N_max + TKT - 1) / TKT;   // positions per lane
    if (P <= 32) hipLaunchKernelGGL(topk_il_kernel<1>, dim3(a.B), dim3(TKT), 0, s, a);
    else if (P <= 64) hipLaunchKernelGGL(topk_il_kernel<2>, dim3(a.B), dim3(TKT), 0, s, a);
    else if (P <= 128) hipLaunchKernelGGL(topk_il_kernel<4>, dim3(a.B), dim3(TKT), 0, s, a);
    else hipLaunchKernelGGL(topk_kernel, dim3(a.B), dim3(TKT), 0, s, a);
    return hipGetLastError();
}

}  // namespace dustin
