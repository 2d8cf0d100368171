// Sparse (and dense) verification attention for gfx950.
//
// Computes, for every sequence b, KV head g and the R = w * G query rows that
// share g (the w window tokens times the G query heads of the group), the
// softmax attention over the selected history rows only: Stage 2 of the
// Dustin blog's Fig. 5 ("compressed KV").  Without an index list the same
// kernel streams every row j < n_b (the "Full Cache" baseline of Fig. 7).
//
// Work decomposition: one 64-lane work-group per (b, g, token split).  The
// split's K and V rows are gathered tile by tile (32 tokens) straight into
// LDS with global->LDS DMA (16 B per lane), NBUF tiles deep, so the HBM
// gather of later tiles overlaps the MFMA work on the current one.  Rows are
// stored with a 16-byte-chunk XOR swizzle so that both the K operand reads
// (ds_read_b128) and the transposed V reads (ds_read_b64_tr_b16) are free of
// bank conflicts.
//
//   S^T[token][row] = K_tile . Q^T      v_mfma_f32_16x16x32_bf16, fp32 acc
//   online softmax over tokens (exp2 domain, per-row running max)
//   O^T[d][row]    += V_tile^T . P^T    P rounded to bf16 for the MFMA
//
// Splits of one (b, g) are merged by the last work-group to finish (an
// atomic arrival counter in the workspace, reset to zero afterwards), so the
// whole call is one kernel launch.  The merge order is fixed, which keeps the
// output bitwise deterministic.
//
// A float32 variant (plain VALU arithmetic, 256 lanes per work-group) serves
// float32 caches with the same split/merge scheme.

#include "common.h"
#include "internal.h"

namespace dustin {

// All-zero stand-in for absent rows (masked tokens still go through the DMA
// so that every lane of every tile has a defined, finite source).
__device__ __align__(256) uint8_t g_zero_row[1024] = {0};

// Physical row of logical position j of sequence b (j already in [0, n_b)),
// or -1 if the page table entry is out of range.
__device__ __forceinline__ int phys_row(const KvView &kv, int b, int j) {
    if (kv.page_size == 0) return b * kv.N_max + j;
    const int pg = kv.page_table[(int64_t)b * kv.max_pages + (j >> 4)];
    if (pg < 0 || pg >= kv.num_pages) return -1;
    return pg * 16 + (j & 15);
}

// 16-byte-chunk swizzle of row r of a tile.  D = 128: a bijection on the low
// four bits (16 rows at one chunk -> 16 distinct chunk slots; four
// consecutive rows -> four distinct chunk pairs).  D = 64: two rows share a
// 64-bank span, so the swizzle acts on r >> 1.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) {
        const int x = r & 15;
        return ((x << 1) | (x >> 3)) & 15;
    } else {
        const int x = (r >> 1) & 7;
        return ((x << 1) | (x >> 2)) & 7;
    }
}

__device__ __forceinline__ int seq_len(const KvView &kv, int b) {
    return min(max(kv.seq_lens[b], 0), kv.N_max);
}

// Merge the split partials of (b, g) and write the output rows.  Executed by
// one wave (64 lanes).
template <bool F32OUT, int D>
__device__ void merge_splits(const AttnArgs &a, int bg, int b, int g, int lane) {
    const size_t pb = (size_t)bg * a.splits * a.rpad;
    for (int r = 0; r < a.R; ++r) {
        float mx = kNegInf;
        for (int s = lane; s < a.splits; s += 64) mx = fmaxf(mx, a.part_m[pb + (size_t)s * a.rpad + r]);
        mx = wave_max(mx);
        const float muse = (mx == kNegInf) ? 0.f : mx;
        float L = 0.f;
        for (int s = lane; s < a.splits; s += 64) {
            const size_t o = pb + (size_t)s * a.rpad + r;
            L += a.part_l[o] * exp2f(a.part_m[o] - muse);
        }
        L = wave_sum(L);
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        const int sq = r / a.G, gh = r - sq * a.G;
        const size_t orow = (((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh) * D;
        for (int d = lane * 2; d < D; d += 128) {
            float acc0 = 0.f, acc1 = 0.f;
            for (int s = 0; s < a.splits; ++s) {
                const size_t o = pb + (size_t)s * a.rpad + r;
                const float ws = exp2f(a.part_m[o] - muse);
                const float *po = a.part_o + o * D + d;
                acc0 += ws * po[0];
                acc1 += ws * po[1];
            }
            acc0 *= inv;
            acc1 *= inv;
            if constexpr (F32OUT) {
                float *op = (float *)a.out + orow + d;
                op[0] = acc0;
                op[1] = acc1;
            } else {
                uint32_t packed = f32_to_bf16_bits(acc0) | ((uint32_t)f32_to_bf16_bits(acc1) << 16);
                *(uint32_t *)((uint16_t *)a.out + orow + d) = packed;
            }
        }
        if (a.lse && lane == 0) {
            a.lse[((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh] =
                (L > 0.f) ? (mx + __log2f(L)) * kLn2 : kNegInf;
        }
    }
}

// Arrival on the (b, g) counter after this work-group's partial is stored.
// Returns true for the last of the a.splits arrivals.
__device__ __forceinline__ bool arrive_last(const AttnArgs &a, int bg, int lane) {
    __threadfence();
    int prev = 0;
    if (lane == 0) prev = atomicAdd(&a.counters[bg], 1);
    prev = __shfl(prev, 0, 64);
    if (prev != a.splits - 1) return false;
    __threadfence();
    return true;
}

// --------------------------------------------------------------- bf16 / MFMA
template <int D, int RB, int NBUF>
__global__ __launch_bounds__(64) void attn_bf16_kernel(AttnArgs a) {
    constexpr int T = kAttnTile;
    constexpr int ROWB = D * 2;       // bytes of one head row
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;     // rows per DMA instruction
    constexpr int NI = T / RPI;       // DMA instructions per K (or V) tile
    constexpr int TB = T * ROWB;      // bytes of one K tile
    constexpr int KK = D / 32;        // k-steps of the QK^T MFMA
    constexpr int DT = D / 16;        // 16-wide d tiles of the PV MFMA
    static_assert(NI * 1024 == TB, "tile / DMA geometry");

    __shared__ __attribute__((aligned(1024))) uint8_t sm[NBUF][2][TB];
    __shared__ int rows[kAttnMaxTps];

    const int lane = threadIdx.x;
    const int split = blockIdx.x % a.splits;
    const int bg = blockIdx.x / a.splits;
    const int b = bg / a.kv.Hkv, g = bg - (bg / a.kv.Hkv) * a.kv.Hkv;

    const int nb = seq_len(a.kv, b);
    const int cnt = a.idx ? min(max(a.count[b], 0), a.k) : nb;
    const int t0 = split * a.tps;
    const int ntok = max(0, min(cnt, t0 + a.tps) - t0);

    for (int t = lane; t < ntok; t += 64) {
        const int j = a.idx ? a.idx[(int64_t)b * a.k + t0 + t] : t0 + t;
        rows[t] = (j >= 0 && j < nb) ? phys_row(a.kv, b, j) : -1;
    }
    __syncthreads();

    // Q^T operand fragments: lane holds row (lane & 15), d slice (lane >> 4) * 8.
    bf16x8 qf[RB][KK];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rb * 16 + (lane & 15);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (r < a.R) {
                const int sq = r / a.G, gh = r - (r / a.G) * a.G;
                const uint16_t *qp = (const uint16_t *)a.q +
                    (((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh) * D + kk * 32 + (lane >> 4) * 8;
                qf[rb][kk] = *(const bf16x8 *)qp;
            } else {
                for (int i = 0; i < 8; ++i) qf[rb][kk][i] = (__bf16)0.f;
            }
        }
    }

    f32x4 o[RB][DT];
    float mrow[RB], lsum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        mrow[rb] = kNegInf;
        lsum[rb] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const char *kbase = a.kv.k;
    const char *vbase = a.kv.v;
    const size_t head_off = (size_t)g * ROWB;
    const size_t row_stride = (size_t)a.kv.Hkv * ROWB;

    auto issue = [&](int tile, int buf) {
        const int tb = tile * T;
#pragma unroll
        for (int c = 0; c < NI; ++c) {
            const int rho = c * RPI + lane / CPR;
            const int chunk = (lane % CPR) ^ swz<D>(rho);
            const int t = tb + rho;
            const int r = (t < ntok) ? rows[t] : -1;
            const char *kp, *vp;
            if (r >= 0) {
                const size_t off = (size_t)r * row_stride + head_off + chunk * 16;
                kp = kbase + off;
                vp = vbase + off;
            } else {
                kp = vp = (const char *)g_zero_row + chunk * 16;
            }
            dma16(kp, &sm[buf][0][c * 1024]);
            dma16(vp, &sm[buf][1][c * 1024]);
        }
    };

    auto compute = [&](int tile, int buf) {
        const uint8_t *kt = sm[buf][0];
        const uint8_t *vt = sm[buf][1];
        const int tb = tile * T;
        f32x4 st[2][RB];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) st[ts][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int rho = ts * 16 + (lane & 15);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int chunk = kk * 4 + (lane >> 4);
                const bf16x8 kf = *(const bf16x8 *)(kt + rho * ROWB + ((chunk ^ swz<D>(rho)) << 4));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    st[ts][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][kk], st[ts][rb], 0, 0, 0);
            }
        }
        // validity of the 8 tokens this lane holds: t = tb + ts*16 + (lane>>4)*4 + j
        bool valid[2][4];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = tb + ts * 16 + (lane >> 4) * 4 + j;
                valid[ts][j] = (t < ntok) && (rows[t] >= 0);
            }
        bf16x8 pf[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float mx = kNegInf;
#pragma unroll
            for (int ts = 0; ts < 2; ++ts)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float s = valid[ts][j] ? st[ts][rb][j] * a.scale_log2 : kNegInf;
                    st[ts][rb][j] = s;
                    mx = fmaxf(mx, s);
                }
            mx = group4_max(mx);
            const float mnew = fmaxf(mrow[rb], mx);
            const float muse = (mnew == kNegInf) ? 0.f : mnew;
            const float alpha = exp2f(mrow[rb] - muse);
            mrow[rb] = mnew;
            float ps = 0.f;
#pragma unroll
            for (int ts = 0; ts < 2; ++ts)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = exp2f(st[ts][rb][j] - muse);
                    ps += p;
                    pf[rb][ts * 4 + j] = (__bf16)p;
                }
            lsum[rb] = lsum[rb] * alpha + ps;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[rb][dt] *= alpha;
        }
        // PV: V^T fragment via two transposed LDS reads per 16-wide d tile.
        // Rows rho0 and rho0 + 16 share their swizzle, so the second read of
        // each pair is the first address plus 16 rows.
        const int q4 = lane >> 4, sl = lane & 15;
        const int rho0 = 4 * q4 + (sl >> 2);
        const uint32_t vrow = lds_addr(vt) + rho0 * ROWB;
        uint32_t vaddr[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int dcol = dt * 16 + (sl & 3) * 4;
            vaddr[dt] = vrow + (((dcol >> 3) ^ swz<D>(rho0)) << 4) + (dcol & 7) * 2;
        }
        s16x4 vlo[DT], vhi[DT];
        if constexpr (DT == 8) {
            ds_read_tr16_x8<16 * ROWB>(vaddr, vlo, vhi);
        } else {
            ds_read_tr16_x4<16 * ROWB>(vaddr, vlo, vhi);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            s16x8 vv;
            vv[0] = vlo[dt][0]; vv[1] = vlo[dt][1]; vv[2] = vlo[dt][2]; vv[3] = vlo[dt][3];
            vv[4] = vhi[dt][0]; vv[5] = vhi[dt][1]; vv[6] = vhi[dt][2]; vv[7] = vhi[dt][3];
            const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                o[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb], o[rb][dt], 0, 0, 0);
        }
    };

    const int ntiles = (ntok + T - 1) / T;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
        if (i < ntiles) issue(i, i);
    for (int i = 0; i < ntiles; ++i) {
        const int nxt = i + NBUF - 1;
        if (nxt < ntiles) issue(nxt, nxt % NBUF);
        const int ahead = min(ntiles - 1 - i, NBUF - 1);
        // wait until tile i's 2*NI DMA operations have landed
        if constexpr (NBUF >= 4) {
            if (ahead >= 3) { wait_vmcnt<3 * 2 * NI>(); goto ready; }
        }
        if constexpr (NBUF >= 3) {
            if (ahead >= 2) { wait_vmcnt<2 * 2 * NI>(); goto ready; }
        }
        if (ahead >= 1) { wait_vmcnt<2 * NI>(); goto ready; }
        wait_vmcnt<0>();
    ready:
        compute(i, i % NBUF);
    }

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lsum[rb] = group4_sum(lsum[rb]);

    if (a.splits == 1) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = rb * 16 + (lane & 15);
            if (r >= a.R) continue;
            const int sq = r / a.G, gh = r - (r / a.G) * a.G;
            const size_t orow = (((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh) * D;
            const float inv = (lsum[rb] > 0.f) ? 1.f / lsum[rb] : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 16 + (lane >> 4) * 4;
                uint32_t lo = f32_to_bf16_bits(o[rb][dt][0] * inv) | ((uint32_t)f32_to_bf16_bits(o[rb][dt][1] * inv) << 16);
                uint32_t hi = f32_to_bf16_bits(o[rb][dt][2] * inv) | ((uint32_t)f32_to_bf16_bits(o[rb][dt][3] * inv) << 16);
                uint32_t *op = (uint32_t *)((uint16_t *)a.out + orow + d);
                op[0] = lo;
                op[1] = hi;
            }
            if (a.lse && lane < 16)
                a.lse[((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh] =
                    (lsum[rb] > 0.f) ? (mrow[rb] + __log2f(lsum[rb])) * kLn2 : kNegInf;
        }
        return;
    }

    const size_t pb = ((size_t)bg * a.splits + split) * a.rpad;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rb * 16 + (lane & 15);
        if (lane < 16) {
            a.part_m[pb + r] = mrow[rb];
            a.part_l[pb + r] = lsum[rb];
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *(f32x4 *)(a.part_o + (pb + r) * D + dt * 16 + (lane >> 4) * 4) = o[rb][dt];
    }
    if (!arrive_last(a, bg, lane)) return;
    merge_splits<false, D>(a, bg, b, g, lane);
    if (lane == 0) a.counters[bg] = 0;
}

// --------------------------------------------------------------- float32 / VALU
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
    constexpr int T = kAttnTile;
    __shared__ float ks[T][D + 1];
    __shared__ float vs[T][D];
    __shared__ float qs[64][D + 1];
    __shared__ float ps[64][T + 1];
    __shared__ float alpha_s[64];
    __shared__ float m_s[64];
    __shared__ float l_s[64];
    __shared__ int rows[kAttnMaxTps];

    const int tid = threadIdx.x;
    const int split = blockIdx.x % a.splits;
    const int bg = blockIdx.x / a.splits;
    const int b = bg / a.kv.Hkv, g = bg - (bg / a.kv.Hkv) * a.kv.Hkv;
    const int nb = seq_len(a.kv, b);
    const int cnt = a.idx ? min(max(a.count[b], 0), a.k) : nb;
    const int t0 = split * a.tps;
    const int ntok = max(0, min(cnt, t0 + a.tps) - t0);
    const int R = a.R;

    for (int t = tid; t < ntok; t += 256) {
        const int j = a.idx ? a.idx[(int64_t)b * a.k + t0 + t] : t0 + t;
        rows[t] = (j >= 0 && j < nb) ? phys_row(a.kv, b, j) : -1;
    }
    for (int e = tid; e < R * D; e += 256) {
        const int r = e / D, d = e - (e / D) * D;
        const int sq = r / a.G, gh = r - (r / a.G) * a.G;
        qs[r][d] = ((const float *)a.q)[(((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh) * D + d];
    }
    if (tid < 64) {
        m_s[tid] = kNegInf;
        l_s[tid] = 0.f;
    }
    constexpr int PER = (64 * D + 255) / 256;
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    __syncthreads();

    const size_t row_stride = (size_t)a.kv.Hkv * D;
    const float *kb = (const float *)a.kv.k;
    const float *vb = (const float *)a.kv.v;
    for (int tb = 0; tb < ntok; tb += T) {
        for (int e = tid; e < T * D; e += 256) {
            const int t = e / D, d = e - (e / D) * D;
            const int r = (tb + t < ntok) ? rows[tb + t] : -1;
            float kv = 0.f, vv = 0.f;
            if (r >= 0) {
                const size_t off = (size_t)r * row_stride + (size_t)g * D + d;
                kv = kb[off];
                vv = vb[off];
            }
            ks[t][d] = kv;
            vs[t][d] = vv;
        }
        __syncthreads();
        for (int e = tid; e < R * T; e += 256) {
            const int r = e / T, t = e - (e / T) * T;
            const int tr = (tb + t < ntok) ? rows[tb + t] : -1;
            float s = 0.f;
            for (int d = 0; d < D; ++d) s += qs[r][d] * ks[t][d];
            ps[r][t] = (tr >= 0) ? s * a.scale_log2 : kNegInf;
        }
        __syncthreads();
        if (tid < R) {
            float mx = kNegInf;
            for (int t = 0; t < T; ++t) mx = fmaxf(mx, ps[tid][t]);
            const float mold = m_s[tid];
            const float mnew = fmaxf(mold, mx);
            const float muse = (mnew == kNegInf) ? 0.f : mnew;
            const float al = exp2f(mold - muse);
            float sum = 0.f;
            for (int t = 0; t < T; ++t) {
                const float p = exp2f(ps[tid][t] - muse);
                ps[tid][t] = p;
                sum += p;
            }
            m_s[tid] = mnew;
            l_s[tid] = l_s[tid] * al + sum;
            alpha_s[tid] = al;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + i * 256;
            if (e < R * D) {
                const int r = e / D, d = e - (e / D) * D;
                float s = acc[i] * alpha_s[r];
                for (int t = 0; t < T; ++t) s += ps[r][t] * vs[t][d];
                acc[i] = s;
            }
        }
        __syncthreads();
    }

    if (a.splits == 1) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + i * 256;
            if (e < R * D) {
                const int r = e / D, d = e - (e / D) * D;
                const int sq = r / a.G, gh = r - (r / a.G) * a.G;
                const float L = l_s[r];
                ((float *)a.out)[(((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh) * D + d] =
                    (L > 0.f) ? acc[i] / L : 0.f;
            }
        }
        if (a.lse && tid < R) {
            const int sq = tid / a.G, gh = tid - (tid / a.G) * a.G;
            const float L = l_s[tid];
            a.lse[((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh] =
                (L > 0.f) ? (m_s[tid] + __log2f(L)) * kLn2 : kNegInf;
        }
        return;
    }

    const size_t pb = ((size_t)bg * a.splits + split) * a.rpad;
    if (tid < R) {
        a.part_m[pb + tid] = m_s[tid];
        a.part_l[pb + tid] = l_s[tid];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid + i * 256;
        if (e < R * D) {
            const int r = e / D, d = e - (e / D) * D;
            a.part_o[(pb + r) * D + d] = acc[i];
        }
    }
    __syncthreads();
    if (tid >= 64) return;
    if (!arrive_last(a, bg, tid)) return;
    merge_splits<true, D>(a, bg, b, g, tid);
    if (tid == 0) a.counters[bg] = 0;
}

// --------------------------------------------------------------- host side
AttnPlan attn_plan(int B, int w, int Hq, int Hkv, int D, int tokens, bool f32) {
    AttnPlan p{};
    const int G = Hq / Hkv;
    p.rows = w * G;
    p.rb = (p.rows + 15) / 16;
    p.rpad = p.rb * 16;
    const long groups = (long)B * Hkv;
    const int tok = tokens > 0 ? tokens : 1;
    // Aim for ~3 co-resident 64-lane work-groups per CU on a 256-CU part,
    // with at least one 32-token tile per split and at most kAttnMaxTps
    // tokens per split.  The plan depends on shapes only, so workspace sizes
    // can be queried without a device.
    (void)f32;
    const long target = 768;
    long splits = (target + groups - 1) / groups;
    const long max_by_tiles = (tok + kAttnTile - 1) / kAttnTile;
    if (splits > max_by_tiles) splits = max_by_tiles;
    if (splits < 1) splits = 1;
    long tps = (tok + splits - 1) / splits;
    tps = (tps + kAttnTile - 1) / kAttnTile * kAttnTile;
    if (tps > kAttnMaxTps) tps = kAttnMaxTps;
    splits = (tok + tps - 1) / tps;
    p.splits = (int)splits;
    p.tps = (int)tps;
    size_t off = align_up((size_t)groups * sizeof(int32_t), 256);
    if (p.splits > 1) {
        const size_t nrow = (size_t)groups * p.splits * p.rpad;
        p.off_m = off;
        off = align_up(off + nrow * sizeof(float), 256);
        p.off_l = off;
        off = align_up(off + nrow * sizeof(float), 256);
        p.off_o = off;
        off = align_up(off + nrow * D * sizeof(float), 256);
    } else {
        p.off_m = p.off_l = p.off_o = off;
    }
    p.ws_bytes = off;
    return p;
}

template <int D, int RB>
static hipError_t launch_bf16(const AttnArgs &a, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((attn_bf16_kernel<D, RB, 3>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
    const dim3 grid((unsigned)((size_t)a.kv.B * a.kv.Hkv * p.splits));
    if (a.kv.f32) {
        switch (a.kv.D) {
            case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(256), 0, s, a); break;
            case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, s, a); break;
            case 128: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.kv.D == 128) {
        switch (p.rb) {
            case 1: return launch_bf16<128, 1>(a, grid, s);
            case 2: return launch_bf16<128, 2>(a, grid, s);
            case 3: return launch_bf16<128, 3>(a, grid, s);
            case 4: return launch_bf16<128, 4>(a, grid, s);
        }
    } else if (a.kv.D == 64) {
        switch (p.rb) {
            case 1: return launch_bf16<64, 1>(a, grid, s);
            case 2: return launch_bf16<64, 2>(a, grid, s);
            case 3: return launch_bf16<64, 3>(a, grid, s);
            case 4: return launch_bf16<64, 4>(a, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dustin
