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
// the unsigned order of the bits is the numeric order): three passes of
// 11/11/10-bit digits with the histogram in LDS find the k-th largest key T
// and how many keys equal to T are needed; one ordered pass then takes every
// key above T plus the lowest positions among the keys equal to T.  Position
// j is always handled by lane j mod 1024, so the per-position tier flags need
// no synchronisation beyond the block barriers.

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
// use the kernel above): lane t owns the P = ceil(n
// / 1024) consecutive positions [t P, t P + P) and keeps their draft / target
// selection flags as bit masks in registers, so every ordered step (ties at
// the threshold, the ascending compaction) needs a single block-wide prefix
// count instead of one per 1024 positions, and no flag array goes to memory.

// Exclusive prefix sum of v over the work-group in lane order, plus the total.
__device__ __forceinline__ int block_prefix(int v, int &total, TopkShared &sh) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
    for (int w = 0; w < TKW; ++w) {
        const int c = sh.wave_tot[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// Select the K largest candidate keys of this lane's range (candidates: the
// bits of cm), setting their bits in `sel`.  Requires 1 <= K <= number of
// candidates over the work-group (ncand).  Keys are read 32 at a time with
// all loads in flight together; for short ranges (MW == 1) they are read
// once and kept in registers for all passes.
template <int MW>
__device__ __forceinline__ void load_keys(const float *sc, int j0, int P, int w, uint32_t (&kw)[32]) {
#pragma unroll
    for (int bit = 0; bit < 32; ++bit) {
        const int i = w * 32 + bit;
        kw[bit] = (i < P) ? __float_as_uint(sc[j0 + i]) : 0u;
    }
}

template <int MW>
__device__ __forceinline__ void select_top_regs(const float *sc, int j0, int P, const uint32_t (&cm)[MW],
                                                uint32_t (&sel)[MW], int K, int ncand, TopkShared &sh) {
    const int tid = threadIdx.x;
    if (K >= ncand) {
#pragma unroll
        for (int w = 0; w < MW; ++w) sel[w] = cm[w];
        return;
    }
    constexpr bool CACHE = MW == 1;
    uint32_t kc[CACHE ? MW : 1][32];
    if constexpr (CACHE) {
#pragma unroll
        for (int w = 0; w < MW; ++w) load_keys<MW>(sc, j0, P, w, kc[w]);
    }
    auto each_word = [&](auto &&f) {
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            if (w * 32 >= P) break;
            if constexpr (CACHE) {
                f(w, kc[w]);
            } else {
                uint32_t kw[32];
                load_keys<MW>(sc, j0, P, w, kw);
                f(w, kw);
            }
        }
    };
    uint32_t prefix = 0, mask = 0;
    int remaining = K;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int sh_ = pass == 0 ? 21 : (pass == 1 ? 10 : 0);   // 11 / 11 / 10-bit digits
        const int wd = pass == 2 ? 10 : 11;
        const uint32_t dmask = (1u << wd) - 1u;
        const int nbins = 1 << wd;
        for (int i = tid; i < nbins; i += TKT) sh.hist[i] = 0;
        __syncthreads();
        each_word([&](int w, const uint32_t (&kw)[32]) {
#pragma unroll
            for (int bit = 0; bit < 32; ++bit)
                if (((cm[w] >> bit) & 1u) && (kw[bit] & mask) == prefix) atomicAdd(&sh.hist[(kw[bit] >> sh_) & dmask], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            const int lane = tid;
            const int per = nbins / 64;
            int local = 0;
            for (int i = 0; i < per; ++i) local += (int)sh.hist[lane * per + i];
            int incl = local;   // inclusive suffix sum over lanes >= lane
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
    // keys above the threshold key all go in; of the keys equal to it, the
    // lowest positions fill the remaining `need` places
    const uint32_t thr = prefix;
    const int need = remaining;
    int ties = 0;
    uint32_t tie[MW];
#pragma unroll
    for (int w = 0; w < MW; ++w) sel[w] = tie[w] = 0;
    each_word([&](int w, const uint32_t (&kw)[32]) {
        uint32_t m = 0, t = 0;
#pragma unroll
        for (int bit = 0; bit < 32; ++bit) {
            const bool c = (cm[w] >> bit) & 1u;
            m |= (uint32_t)(c && kw[bit] > thr) << bit;
            t |= (uint32_t)(c && kw[bit] == thr) << bit;
        }
        sel[w] = m;
        tie[w] = t;
        ties += __popc(t);
    });
    int tot;
    int rank = block_prefix(ties, tot, sh);
#pragma unroll
    for (int w = 0; w < MW; ++w) {
        uint32_t t = tie[w];
        while (t && rank < need) {   // lowest positions first
            const uint32_t low = t & (0u - t);
            sel[w] |= low;
            t ^= low;
            ++rank;
        }
    }
}

template <int MW>
__global__ __launch_bounds__(TKT) void topk_regs_kernel(TopkArgs a) {
    __shared__ TopkShared sh;
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

    const int P = (n + TKT - 1) / TKT;
    const int j0 = tid * P;
    const int Pl = max(0, min(P, n - j0));   // positions this lane owns
    uint32_t cm[MW], dsel[MW], tsel[MW];     // candidates, draft tier, target tier
#pragma unroll
    for (int w = 0; w < MW; ++w) {
        uint32_t m = 0;
#pragma unroll
        for (int bit = 0; bit < 32; ++bit) {
            const int i = w * 32 + bit, j = j0 + i;
            m |= (uint32_t)(i < Pl && !(j < se || j >= wb)) << bit;
        }
        cm[w] = m;
        dsel[w] = tsel[w] = 0;
    }
    if (m_eff > 0) select_top_regs<MW>(a.s_draft + (int64_t)(a.d_mod ? b % a.d_mod : b) * a.N_max, j0, Pl, cm, dsel, m_eff, rest, sh);
#pragma unroll
    for (int w = 0; w < MW; ++w) cm[w] &= ~dsel[w];
    if (t_cnt > 0) select_top_regs<MW>(a.s_target + (int64_t)(a.t_mod ? b % a.t_mod : b) * a.N_max, j0, Pl, cm, tsel, t_cnt, rest - m_eff, sh);

    // ascending compaction: one prefix count over the lanes' ranges
    int mine = 0;
    for (int i = 0; i < Pl; ++i) {
        const int j = j0 + i;
        mine += (j < se || j >= wb);
    }
#pragma unroll
    for (int w = 0; w < MW; ++w) mine += __popc(dsel[w] | tsel[w]);
    int written;
    int pos = block_prefix(mine, written, sh);
    int32_t *idx = a.idx + (int64_t)b * a.k;
    int8_t *tier = a.tier ? a.tier + (int64_t)b * a.k : nullptr;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
        for (int bit = 0; bit < 32; ++bit) {
            const int i = w * 32 + bit;
            if (i >= Pl) break;
            const int j = j0 + i;
            int t = -1;
            if (j < se || j >= wb) t = 0;
            else if ((dsel[w] >> bit) & 1u) t = 1;
            else if ((tsel[w] >> bit) & 1u) t = 2;
            if (t >= 0) {
                if (pos < a.k) {
                    idx[pos] = j;
                    if (tier) tier[pos] = (int8_t)t;
                }
                ++pos;
            }
        }
    }
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
    if (P <= 32) hipLaunchKernelGGL(topk_regs_kernel<1>, dim3(a.B), dim3(TKT), 0, s, a);
    else if (P <= 64) hipLaunchKernelGGL(topk_regs_kernel<2>, dim3(a.B), dim3(TKT), 0, s, a);
    else if (P <= 128) hipLaunchKernelGGL(topk_regs_kernel<4>, dim3(a.B), dim3(TKT), 0, s, a);
    else hipLaunchKernelGGL(topk_kernel, dim3(a.B), dim3(TKT), 0, s, a);
    return hipGetLastError();
}

}  // namespace dustin
