// Sparse (and dense) verification attention for gfx950.
//
// Computes, for every sequence b, KV head g and the R = w * G query rows that
// share g (the w window tokens times the G query heads of the group), the
// softmax attention over the selected history rows only: Stage 2 of the
// Dustin blog's Fig. 5 ("compressed KV").  Without an index list the same
// kernel streams every row j < n_b (the "Full Cache" baseline of Fig. 7).
//
// Work decomposition: one work-group per (b, g, token split), sized to fill
// one CU (8 waves, about 130 KiB of LDS), with the splits planned so that
// the grid is about one group per CU.  The split's K and V rows are gathered
// tile by tile straight into an LDS ring with global->LDS DMA (16 B per
// lane), several tiles deep, so the HBM gather of later tiles overlaps the
// MFMA work on the current one.  Rows are stored with a 16-byte-chunk XOR
// swizzle so that both the K operand reads (ds_read_b128) and the transposed
// V reads (ds_read_b64_tr_b16) are free of bank conflicts.
//
//   S^T[token][row] = K_tile . Q^T      v_mfma_f32_16x16x32_bf16, fp32 acc
//   online softmax over tokens (exp2 domain, per-row running max)
//   O^T[d][row]    += V_tile^T . P^T    P rounded to bf16 for the MFMA
//
// Splits of one (b, g) are merged inside the same launch through an arrival
// counter in the workspace (reset to zero afterwards): a split that finds all
// the others already published merges at once, otherwise the last one to
// arrive does.  The merge order is fixed, which keeps the output bitwise
// deterministic.
//
// A float32 variant (plain VALU arithmetic, 256 lanes per work-group) serves
// float32 caches with the same split/merge scheme.

#include "attn.h"
#include "common.h"

namespace dustin {

// Phase trace (builds with DUSTIN_ATTN_TRACE only; the library proper has
// none of it): thread 0 of every work-group of the bf16 kernel records the
// 100 MHz real-time counter at kernel entry, when the row table is ready,
// when the first tile has landed, at the end of the token loop, after the
// split partial is stored, after the split handshake and at exit, plus the
// path it took (0 one split, 1 merged at once, 2 merged after arriving last,
// 3 published only) and the XCD it ran on.  Launch l fills row l mod
// kTraceLaunches of g_attn_trace.
#ifdef DUSTIN_ATTN_TRACE
constexpr int kTraceLaunches = 80, kTraceGroups = 1024;
__device__ unsigned long long g_attn_trace[kTraceLaunches][kTraceGroups][8];
__device__ __forceinline__ unsigned long long trace_clock() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ unsigned trace_xcc() {
    unsigned v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v;
}
#define ATTN_TRACE_DECL unsigned long long trace_t[7] = {trace_clock(), 0, 0, 0, 0, 0, 0}
#define ATTN_TRACE(i) (trace_t[i] = trace_clock())
#define ATTN_TRACE_DUMP(path)                                                                        \
    do {                                                                                             \
        if (threadIdx.x == 0 && blockIdx.x < kTraceGroups) {                                         \
            unsigned long long *o_ = g_attn_trace[a.trace_slot % kTraceLaunches][blockIdx.x];        \
            for (int i_ = 0; i_ < 6; ++i_) o_[i_] = trace_t[i_];                                     \
            o_[6] = trace_clock();                                                                   \
            o_[7] = (unsigned long long)(path) | ((unsigned long long)trace_xcc() << 8);             \
        }                                                                                            \
    } while (0)
#else
#define ATTN_TRACE_DECL
#define ATTN_TRACE(i)
#define ATTN_TRACE_DUMP(path)
#endif

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
// 64-bank span, so the swizzle acts on r >> 1.  D = 32: four rows of four
// chunks share a span; rows r and r + 4k take chunk slots c ^ k, so 16
// consecutive rows at one chunk fill the 16 bank groups of four spans.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) {
        const int x = r & 15;
        return ((x << 1) | (x >> 3)) & 15;
    } else if constexpr (D == 32) {
        return (r >> 2) & 3;
    } else {
        const int x = (r >> 1) & 7;
        return ((x << 1) | (x >> 2)) & 7;
    }
}

__device__ __forceinline__ int seq_len(const KvView &kv, int b) {
    return min(max(kv.seq_lens[b], 0), kv.N_max);
}

// Merge the split partials of (b, g) and write the output rows, using NT
// threads.  Each thread owns one (row, eighth of d) slice and folds the
// splits in with a running maximum, so every load is independent of the
// arithmetic and the merge costs about one memory round trip.
template <bool F32OUT, int D, int NT>
__device__ void merge_splits(const AttnArgs &a, int bg, int b, int g, int tid) {
    constexpr int PART = D / 8;    // floats per (row, part) slice
    constexpr int NC = PART / 4;   // float4 chunks per slice
    // The partials were stored write-through (st_agent) before their
    // writers' arrivals; read them back device-coherently.
    const size_t pb = (size_t)bg * a.splits * a.rpad;
    const uint32_t nml = (uint32_t)(a.splits * a.rpad * sizeof(float));
    const __amdgpu_buffer_rsrc_t pm = coherent_rsrc(a.part_m + pb, nml);
    const __amdgpu_buffer_rsrc_t pl = coherent_rsrc(a.part_l + pb, nml);
    const __amdgpu_buffer_rsrc_t po = coherent_rsrc(a.part_o + pb * D, nml * D);
    for (int e = tid; e < a.R * 8; e += NT) {
        const int r = e >> 3, h = e & 7;
        float M = kNegInf, L = 0.f;
        f32x4 acc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int s = 0; s < a.splits; ++s) {
            const uint32_t o = (uint32_t)(s * a.rpad + r);
            const float ms = ld_coherent(pm, o * 4u), ls = ld_coherent(pl, o * 4u);
            f32x4 v[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) v[c] = ld_coherent4(po, (o * D + h * PART + 4 * c) * 4u);
            const float Mn = fmaxf(M, ms);
            const float mu = (Mn == kNegInf) ? 0.f : Mn;
            const float so = exp2f(M - mu), sn = exp2f(ms - mu);
            L = L * so + ls * sn;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c] = acc[c] * so + v[c] * sn;
            M = Mn;
        }
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        const int sq = r / a.G, gh = r - (r / a.G) * a.G;
        const size_t hrow = ((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh;
        const size_t orow = hrow * D + h * PART;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const f32x4 v = acc[c] * inv;
            if constexpr (F32OUT) {
                *(f32x4 *)((float *)a.out + orow + 4 * c) = v;
            } else {
                uint32_t lo = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
                uint32_t hi = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
                uint32_t *op = (uint32_t *)((uint16_t *)a.out + orow + 4 * c);
                op[0] = lo;
                op[1] = hi;
            }
        }
        if (a.lse && h == 0) a.lse[hrow] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
    }
}

// Split partials are exchanged through device-coherent stores and loads
// (st_agent / ld_agent): a work-group stores its partial, waits for the
// stores to complete, and only then bumps the (b, g) arrival counter; the
// last of the a.splits arrivals merges.  Single-wave variant.
__device__ __forceinline__ bool arrive_last(const AttnArgs &a, int bg, int lane) {
    wait_all_mem();
    int prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(&a.counters[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, 64);
    return prev == a.splits - 1;
}

// --------------------------------------------------------------- bf16 / MFMA
// NW waves share one LDS ring of NBUF tiles of T tokens.  Wave w owns row
// block w % RB (16 query rows) and, of every tile, the 16-token subtiles
// s = w / RB (mod NTH) with NTH = NW / RB: each wave keeps its own running
// softmax state over its share of the tokens, so no score or exponential is
// computed twice; the shares of one row block are folded through LDS at the
// end, every wave folding one slice of the d columns.  Each wave issues
// 1 / NW of every tile's DMA.  One barrier per tile both publishes the tile
// and frees the buffer the next DMA overwrites; it waits only for LDS
// traffic (lds_barrier), so the DMA of later tiles stays in flight.
//
// Per 16-token subtile and row block:
//   S^T = K_sub . Q^T         4 (D = 128) x v_mfma_f32_16x16x32_bf16
//   P   = exp2(S^T - m)       lane holds row (lane & 15), tokens 4*(lane>>4)+j
//   O^T += V_sub^T . P^T      D/16 x v_mfma_f32_16x16x16_bf16; the V operand
//                             comes from one transposed LDS read per d tile.

// Wait until this wave's DMA for the current tile has landed while the
// `ahead` tiles issued after it (PER instructions each) may stay in flight.
template <int A, int PER>
__device__ __forceinline__ void wait_tile(int ahead) {
    if constexpr (A <= 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= A) wait_vmcnt<A * PER>();
        else wait_tile<A - 1, PER>(ahead);
    }
}

template <int D, int RB, int NW>
struct AttnGeom {
    // tokens per tile: at least kAttnTile, 16 per token share of a row block,
    // and one DMA instruction (64 lanes x 16 bytes) per wave for K and for V
    static constexpr int T0 = (16 * NW / RB > kAttnTile) ? 16 * NW / RB : kAttnTile;
    static constexpr int T = (NW * (512 / D) > T0) ? NW * (512 / D) : T0;
    static constexpr int STAGE = 2 * T * D * 2;                                        // K + V bytes per tile
    static constexpr int NBUF = (kAttnRingBytes / STAGE < 8) ? kAttnRingBytes / STAGE : 8;
};

template <int D, int RB, int NW, bool DENSE, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(AttnArgs a) {
    constexpr int T = AttnGeom<D, RB, NW>::T;
    constexpr int NBUF = AttnGeom<D, RB, NW>::NBUF;
    constexpr int ROWB = D * 2;       // bytes of one head row
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;     // rows per DMA instruction
    constexpr int NI = T / RPI;       // DMA instructions per K (or V) tile
    constexpr int TB = T * ROWB;      // bytes of one K tile
    constexpr int KK = D / 32;        // k-steps of the QK^T MFMA
    constexpr int DT = D / 16;        // 16-wide d tiles of the PV MFMA
    constexpr int NT = NW * 64;       // threads per work-group
    constexpr int NTH = NW / RB;      // token shares per row block
    constexpr int NIW = NI / NW;      // DMA instructions per wave per K (or V) tile
    static_assert(RB == 1 || RB == 2 || RB == 4, "row blocks");
    static_assert(NW == 4 || NW == 8, "waves");
    static_assert(NBUF >= 2 && T % 16 == 0 && (T / 16) % NTH == 0, "ring / subtile geometry");
    static_assert(NI * 1024 == TB && NIW >= 1 && NIW * NW == NI, "tile / DMA geometry");

    __shared__ __attribute__((aligned(1024))) uint8_t sm[NBUF][2][TB];
    __shared__ float share_ml[NW][16][2];
    __shared__ int s_flag;
    extern __shared__ int rows[];   // [a.tps] physical rows, sized at launch

    ATTN_TRACE_DECL;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rbw = wave % RB, th = wave / RB;
    const int split = blockIdx.x % a.splits;
    const int bg = blockIdx.x / a.splits;
    const int b = bg / a.kv.Hkv, g = bg - (bg / a.kv.Hkv) * a.kv.Hkv;

    // Every load of the prologue is independent of the others, so they are
    // all in flight together: sequence length and count (scalar), then Q and
    // the split's index entries, with no branch between them: padding rows
    // of Q read row 0 and are zeroed once the loads have landed, and index
    // entries are read through a buffer resource bounded at the row's k
    // entries (entries past the split are masked after).
    const int nb_raw = a.kv.seq_lens[b];
    const int cnt_raw = DENSE ? 0 : a.count[b];
    const int t0 = split * a.tps;

    if (tid == 0) s_flag = 0;
    // Q^T operand fragments of this wave's row block: lane holds row
    // rbw*16 + (lane & 15), d slice kk*32 + (lane >> 4) * 8.
    const int qrow = rbw * 16 + (lane & 15);
    bf16x8 qf[KK];
    {
        const int qr = qrow < a.R ? qrow : 0;
        const int sq = qr / a.G, gh = qr - (qr / a.G) * a.G;
        const uint16_t *qp = (const uint16_t *)a.q +
            (((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh) * D + (lane >> 4) * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const bf16x8 *)(qp + kk * 32);
    }
    constexpr int PER = kAttnMaxTps / NT;
    int jv[PER];
    if constexpr (DENSE) {
#pragma unroll
        for (int i = 0; i < PER; ++i) jv[i] = t0 + tid + NT * i;
    } else {
        const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(a.idx) + (int64_t)b * a.k, (short)0, a.k * 4, 0x00020000);
        // all PER entries are requested (entries past the row's k read 0)
        // before any is masked, so the loads are in flight together
#pragma unroll
        for (int i = 0; i < PER; ++i)
            jv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, (uint32_t)(t0 + tid + NT * i) * 4u, 0, 0);
        // every loaded value is used here, unconditionally: otherwise the
        // compiler sinks a load into the branch of its mask and waits for it
        // there, after the others
#pragma unroll
        for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(jv[i]));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = tid + NT * i;
            jv[i] = (t < a.tps && t0 + t < a.k) ? jv[i] : -1;
        }
    }
    const int nb = min(max(nb_raw, 0), a.kv.N_max);
    // Fused append: split 0 of (b, g) writes head g of the w window rows into
    // cache positions n_b .. n_b + w - 1 (positions past N_max and pages
    // outside [0, num_pages) are skipped, as by the separate append).  The
    // attention itself reads the window rows from k_win / v_win, so no work-
    // group depends on these stores.
    if (CAUSAL && a.k_win != nullptr && split == 0) {
        constexpr int CH16 = D / 8;   // 16-byte chunks of a head row
        for (int e = tid; e < a.w * 2 * CH16; e += NT) {
            const int s = e / (2 * CH16), which = (e / CH16) & 1, ch = e - (e / CH16) * CH16;
            const int pos = nb + s;
            if (pos >= a.kv.N_max) continue;
            int64_t row = (int64_t)b * a.kv.N_max + pos;
            if (a.kv.page_size != 0) {
                const int pg = a.kv.page_table[(int64_t)b * a.kv.max_pages + (pos >> 4)];
                if (pg < 0 || pg >= a.kv.num_pages) continue;
                row = (int64_t)pg * 16 + (pos & 15);
            }
            const int64_t src = ((((int64_t)b * a.w + s) * a.kv.Hkv + g) * D) * 2 + ch * 16;
            const int64_t dst = ((row * a.kv.Hkv + g) * D) * 2 + ch * 16;
            const char *from = which ? a.v_win : a.k_win;
            char *to = const_cast<char *>(which ? a.kv.v : a.kv.k);
            *(u32x4 *)(to + dst) = *(const u32x4 *)(from + src);
        }
    }
    // History tokens of the (b, g) token list come first; with CAUSAL the w
    // draft-window rows (cache positions n_b .. n_b + w - 1) follow them.
    const int hist = DENSE ? nb : min(max(cnt_raw, 0), a.k);
    const int cnt = hist + (CAUSAL ? a.w : 0);
    const int ntok = max(0, min(cnt, t0 + a.tps) - t0);
    const int win_lo = hist - t0;   // local index of the first window token
    lds_barrier();   // s_flag cleared; the loads stay in flight
    bool any_bad = false;
    if (!CAUSAL && a.kv.page_size == 0) {
        // contiguous history-only rows: arithmetic only, no branch per entry
        const int rb0 = b * a.kv.N_max;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (NT * i < a.tps) {   // the same for every lane
                const int t = tid + NT * i;
                const bool ok = jv[i] >= 0 && jv[i] < nb;
                if (t < a.tps) rows[t] = ok ? rb0 + jv[i] : -1;
                any_bad |= t < ntok && !ok;
            }
        }
    } else {   // physical row of every token of the split
        int pos[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = tid + NT * i;
            int p = -1;
            if (t < ntok) {
                if (!CAUSAL || t < win_lo) p = (jv[i] >= 0 && jv[i] < nb) ? jv[i] : -1;
                else p = (nb + t - win_lo < a.kv.N_max) ? nb + t - win_lo : -1;
            }
            pos[i] = p;
        }
        // paged caches: every page-table entry is requested before any is used
        int pg[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i)
            pg[i] = (pos[i] >= 0 && a.kv.page_size != 0) ? a.kv.page_table[(int64_t)b * a.kv.max_pages + (pos[i] >> 4)] : 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = tid + NT * i;
            if (t < ntok) {
                int r = -1;
                if (pos[i] >= 0) {
                    if (a.kv.page_size == 0) r = b * a.kv.N_max + pos[i];
                    else if (pg[i] >= 0 && pg[i] < a.kv.num_pages) r = pg[i] * 16 + (pos[i] & 15);
                }
                // fused append: a present window row is read from the input,
                // coded -2 - s for window step s (-1 stays "absent")
                if (CAUSAL && a.k_win != nullptr && t >= win_lo && r >= 0) r = -2 - (t - win_lo);
                rows[t] = r;
                any_bad |= (r == -1);
            }
        }
    }
    if (any_bad) s_flag = 1;
    // Q fragments and index loads have landed (nothing else is in flight
    // yet), so no wait on them is left for the compiler to place in the loop.
    wait_vmcnt<0>();
    if (qrow >= a.R) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            for (int i = 0; i < 8; ++i) qf[kk][i] = (__bf16)0.f;
    }
    lds_barrier();
    const bool all_rows_valid = (s_flag == 0);
    ATTN_TRACE(1);

    f32x4 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow = kNegInf, lsum = 0.f;

    const char *kbase = a.kv.k;
    const char *vbase = a.kv.v;
    const size_t head_off = (size_t)g * ROWB;
    const size_t row_stride = (size_t)a.kv.Hkv * ROWB;

    auto issue = [&](int tile, int buf) {
        const int tb = tile * T;
        int r[NIW];
#pragma unroll
        for (int ci = 0; ci < NIW; ++ci) {
            const int rho = (wave * NIW + ci) * RPI + lane / CPR;
            const int t = tb + rho;
            r[ci] = (t < ntok) ? rows[t] : -1;
        }
#pragma unroll
        for (int ci = 0; ci < NIW; ++ci) {
            const int c = wave * NIW + ci;
            const int rho = c * RPI + lane / CPR;
            const int chunk = (lane % CPR) ^ swz<D>(rho);
            const char *kp, *vp;
            if (r[ci] >= 0) {
                const size_t off = (size_t)r[ci] * row_stride + head_off + chunk * 16;
                kp = kbase + off;
                vp = vbase + off;
            } else if (CAUSAL && r[ci] <= -2) {   // window row from the fused-append inputs
                const size_t off = ((((size_t)b * a.w + (-2 - r[ci])) * a.kv.Hkv + g) * D) * 2 + chunk * 16;
                kp = a.k_win + off;
                vp = a.v_win + off;
            } else {
                kp = vp = (const char *)g_zero_row + chunk * 16;
            }
            dma16_stream(kp, &sm[buf][0][c * 1024]);
            dma16_stream(vp, &sm[buf][1][c * 1024]);
        }
    };

    // One 16-token subtile `sub` of the tile in `buf`.
    auto compute_sub = [&](int tile, int buf, int sub) {
        const uint8_t *kt = sm[buf][0];
        const uint8_t *vt = sm[buf][1];
        const int tb = tile * T + sub * 16;
        const int krho = sub * 16 + (lane & 15);
        uint32_t kaddr[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int chunk = kk * 4 + (lane >> 4);
            kaddr[kk] = lds_addr(kt) + krho * ROWB + ((chunk ^ swz<D>(krho)) << 4);
        }
        u32x4 kraw[KK];
        ds_read_b128_n(kaddr, kraw);
        bf16x8 kf[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kf[kk] = __builtin_bit_cast(bf16x8, kraw[kk]);
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[kk], st, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) st[j] *= a.scale_log2;
        if (!(all_rows_valid && tb + 16 <= ntok && (!CAUSAL || tb + 16 <= win_lo))) {
            // this lane's query row; window token t_w is visible to window step s iff t_w <= s
            const int sq = (rbw * 16 + (lane & 15)) / a.G;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = tb + (lane >> 4) * 4 + j;
                if (!(t < ntok && rows[t] != -1)) st[j] = kNegInf;
                if (CAUSAL && t >= win_lo && t - win_lo > sq) st[j] = kNegInf;
            }
        }
        float mx = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
        mx = group4_max(mx);
        const float mnew = fmaxf(mrow, mx);
        const float muse = (mnew == kNegInf) ? 0.f : mnew;
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(st[j] - muse);
        if (mnew != mrow) {
            // the running maximum moved for some row of this wave
            const float alpha = __builtin_amdgcn_exp2f(mrow - muse);
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < DT; ++i) o[i] *= alpha;
            mrow = mnew;
        }
        lsum += (p[0] + p[1]) + (p[2] + p[3]);
        s16x4 pf;
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[j] = __builtin_bit_cast(short, (__bf16)p[j]);
        // V^T operand: lane (q = lane>>4, i = lane&15) receives V[tb + 4q + t][d0 + i],
        // t = 0..3, from the 8-byte rows addressed by the lanes 4t + i/4.
        const int sl = lane & 15;
        const int vrho = sub * 16 + 4 * (lane >> 4) + (sl >> 2);
        const uint32_t vrow = lds_addr(vt) + vrho * ROWB;
        uint32_t vaddr[DT];
#pragma unroll
        for (int i = 0; i < DT; ++i) {
            const int dcol = i * 16 + (sl & 3) * 4;
            vaddr[i] = vrow + (((dcol >> 3) ^ swz<D>(vrho)) << 4) + (dcol & 7) * 2;
        }
        s16x4 vf[DT];
        ds_read_tr16_n<DT>(vaddr, vf);
#pragma unroll
        for (int i = 0; i < DT; ++i)
            o[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[i], pf, o[i], 0, 0, 0);
    };

    const int ntiles = (ntok + T - 1) / T;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
        if (i < ntiles) issue(i, i);
    for (int i = 0; i < ntiles; ++i) {
        // own DMA of tile i done (tiles issued after it may stay in flight)
        wait_tile<NBUF - 2, 2 * NIW>(min(ntiles - 1 - i, NBUF - 2));
        lds_barrier();   // tile i visible to all waves; buffer (i-1) free
        if (i == 0) ATTN_TRACE(2);
        {
            const int nxt = i + NBUF - 1;
            if (nxt < ntiles) issue(nxt, nxt % NBUF);
        }
        for (int sub = th; sub < T / 16; sub += NTH) compute_sub(i, i % NBUF, sub);
    }

    ATTN_TRACE(3);
    lsum = group4_sum(lsum);
    // Ring no longer read (every tile's DMA has been waited for): reuse it for
    // the share fold.  LDS-only barriers from here on, so the split
    // handshake's counter load below overlaps the fold.
    lds_barrier();
    int seen = 0;
    if (a.splits > 1 && tid == 0)
        seen = __hip_atomic_load(&a.counters[bg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // Every wave leaves its share (running max, sum and unnormalised O of its
    // rows over its tokens) in LDS.  Then wave (rbw, th) folds the NTH shares
    // of row block rbw, in share order, for the d columns th * DS .. + DS:
    // lane (row = lane & 15, q = lane >> 4) owns E consecutive columns.
    constexpr int SROW = D + 4;   // padded share row (floats): rows start on different banks
    constexpr int DS = D / NTH;
    constexpr int E = DS / 4;
    static_assert(E % 4 == 0, "fold slice");
    static_assert(NW * 16 * SROW * 4 <= NBUF * 2 * TB, "LDS ring reused for the share fold");
    float *shr = (float *)&sm[0][0][0];   // [NW][16][SROW]
    {
        float *my = shr + ((size_t)wave * 16 + (lane & 15)) * SROW + (lane >> 4) * 4;
#pragma unroll
        for (int i = 0; i < DT; ++i) *(f32x4 *)(my + i * 16) = o[i];
        if (lane < 16) {
            share_ml[wave][lane][0] = mrow;
            share_ml[wave][lane][1] = lsum;
        }
    }
    lds_barrier();
    const int row = lane & 15, r = rbw * 16 + row;
    const int d0 = th * DS + (lane >> 4) * E;
    float M = kNegInf, L = 0.f;
    f32x4 acc[E / 4];
#pragma unroll
    for (int c = 0; c < E / 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t2 = 0; t2 < NTH; ++t2) {
        const int w2 = t2 * RB + rbw;
        const float m2 = share_ml[w2][row][0], l2 = share_ml[w2][row][1];
        const float mn = fmaxf(M, m2);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        const float s1 = __builtin_amdgcn_exp2f(M - mu), s2 = __builtin_amdgcn_exp2f(m2 - mu);
        L = L * s1 + l2 * s2;
        const float *src = shr + ((size_t)w2 * 16 + row) * SROW + d0;
#pragma unroll
        for (int c = 0; c < E / 4; ++c) acc[c] = acc[c] * s1 + *(const f32x4 *)(src + 4 * c) * s2;
        M = mn;
    }

    if (a.splits == 1) {
        if (r < a.R) {
            const int sq = r / a.G, gh = r - (r / a.G) * a.G;
            const size_t hrow = ((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh;
            const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
            for (int c = 0; c < E / 4; ++c) {
                uint32_t *op = (uint32_t *)((uint16_t *)a.out + hrow * D + d0 + 4 * c);
                op[0] = f32_to_bf16_bits(acc[c][0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[c][1] * inv) << 16);
                op[1] = f32_to_bf16_bits(acc[c][2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[c][3] * inv) << 16);
            }
            if (a.lse && th == 0 && lane < 16) a.lse[hrow] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
        }
        ATTN_TRACE_DUMP(0);
        return;
    }

    // Split partials (m, l per row; O in thread order).  A split that, when
    // its token loop ended, found every other split of (b, g) already
    // published merges at once: its own partial comes from registers, so it
    // neither waits for its stores nor arrives.  Otherwise it publishes,
    // waits for its stores, and arrives; the last split to arrive merges.
    // Exactly one split merges, always in split order, so the output does
    // not depend on which.
    // The O partial is stored in thread order (chunk c of thread tid at
    // float4 index c * NT + tid): every wave store covers 1 KiB of whole
    // lines, and the merging split reads the other splits' values for its
    // own slice at the same offsets.  (A row-major layout made each lane's
    // 16-byte write-through store land in a line of its own.)
    const size_t pb0 = (size_t)bg * a.splits * a.rpad;   // partial rows of split 0 of (b, g)
    {
        const size_t pb = pb0 + (size_t)split * a.rpad;
        if (th == 0 && lane < 16) {
            st_agent(a.part_m + pb + r, M);
            st_agent(a.part_l + pb + r, L);
        }
        const __amdgpu_buffer_rsrc_t po = coherent_rsrc(a.part_o + pb * D, (uint32_t)(a.rpad * D * sizeof(float)));
#pragma unroll
        for (int c = 0; c < E / 4; ++c) st_coherent4(po, (uint32_t)((c * NT + tid) * 16), acc[c]);
    }
    ATTN_TRACE(4);
    const bool merged_at_once = (seen == a.splits - 1);
    if (tid == 0) s_flag = merged_at_once;
    lds_barrier();   // the partial stores stay in flight
    if (!s_flag) {
        wait_all_mem();
        __syncthreads();
        if (tid == 0)
            s_flag = __hip_atomic_fetch_add(&a.counters[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.splits - 1;
        __syncthreads();
        if (!s_flag) {
            ATTN_TRACE(5);
            ATTN_TRACE_DUMP(3);
            return;
        }
    }
    ATTN_TRACE(5);
    // merge: each lane folds its (row, E columns) slice over the splits, in
    // split order; the partials of up to MB splits are loaded together
    // before any is folded, so a batch costs one memory round trip.
    {
        const uint32_t nml = (uint32_t)(a.splits * a.rpad * sizeof(float));
        const __amdgpu_buffer_rsrc_t pm = coherent_rsrc(a.part_m + pb0, nml);
        const __amdgpu_buffer_rsrc_t pl = coherent_rsrc(a.part_l + pb0, nml);
        const __amdgpu_buffer_rsrc_t po = coherent_rsrc(a.part_o + pb0 * D, nml * D);
        constexpr int MB = 4;
        float Mt = kNegInf, Lt = 0.f;
        f32x4 at[E / 4];
#pragma unroll
        for (int c = 0; c < E / 4; ++c) at[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < a.splits; s0 += MB) {
            float msb[MB], lsb[MB];
            f32x4 vb[MB][E / 4];
#pragma unroll
            for (int q = 0; q < MB; ++q) {
                const int s2 = s0 + q;
                msb[q] = M;
                lsb[q] = L;
#pragma unroll
                for (int c = 0; c < E / 4; ++c) vb[q][c] = acc[c];
                if (s2 < a.splits && s2 != split) {
                    const uint32_t o = (uint32_t)(s2 * a.rpad + r);
                    msb[q] = ld_coherent(pm, o * 4u);
                    lsb[q] = ld_coherent(pl, o * 4u);
                    const uint32_t ob = (uint32_t)(s2 * a.rpad * D) * 4u;
#pragma unroll
                    for (int c = 0; c < E / 4; ++c) vb[q][c] = ld_coherent4(po, ob + (uint32_t)((c * NT + tid) * 16));
                }
            }
#pragma unroll
            for (int q = 0; q < MB; ++q) {
                if (s0 + q >= a.splits) break;
                const float ms = msb[q], ls = lsb[q];
                const float Mn = fmaxf(Mt, ms);
                const float mu = (Mn == kNegInf) ? 0.f : Mn;
                const float so = exp2f(Mt - mu), sn = exp2f(ms - mu);
                Lt = Lt * so + ls * sn;
#pragma unroll
                for (int c = 0; c < E / 4; ++c) at[c] = at[c] * so + vb[q][c] * sn;
                Mt = Mn;
            }
        }
        if (r < a.R) {
            const int sq = r / a.G, gh = r - (r / a.G) * a.G;
            const size_t hrow = ((size_t)b * a.w + sq) * a.Hq + (size_t)g * a.G + gh;
            const float inv = (Lt > 0.f) ? 1.f / Lt : 0.f;
#pragma unroll
            for (int c = 0; c < E / 4; ++c) {
                uint32_t *op = (uint32_t *)((uint16_t *)a.out + hrow * D + d0 + 4 * c);
                op[0] = f32_to_bf16_bits(at[c][0] * inv) | ((uint32_t)f32_to_bf16_bits(at[c][1] * inv) << 16);
                op[1] = f32_to_bf16_bits(at[c][2] * inv) | ((uint32_t)f32_to_bf16_bits(at[c][3] * inv) << 16);
            }
            if (a.lse && th == 0 && lane < 16) a.lse[hrow] = (Lt > 0.f) ? (Mt + __log2f(Lt)) * kLn2 : kNegInf;
        }
    }
    ATTN_TRACE_DUMP(merged_at_once ? 1 : 2);
    if (tid == 0) a.counters[bg] = 0;
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
    // history tokens first; with a.causal the w window rows (positions
    // n_b .. n_b + w - 1) follow, seen causally by the window steps
    const int hist = a.idx ? min(max(a.count[b], 0), a.k) : nb;
    const int cnt = hist + (a.causal ? a.w : 0);
    const int t0 = split * a.tps;
    const int ntok = max(0, min(cnt, t0 + a.tps) - t0);
    const int win_lo = hist - t0;
    const int R = a.R;

    for (int t = tid; t < ntok; t += 256) {
        if (t < win_lo) {
            const int j = a.idx ? a.idx[(int64_t)b * a.k + t0 + t] : t0 + t;
            rows[t] = (j >= 0 && j < nb) ? phys_row(a.kv, b, j) : -1;
        } else {
            const int p = nb + t - win_lo;
            rows[t] = (p < a.kv.N_max) ? phys_row(a.kv, b, p) : -1;
        }
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
            const bool hidden = a.causal && tb + t >= win_lo && tb + t - win_lo > r / a.G;
            ps[r][t] = (tr >= 0 && !hidden) ? s * a.scale_log2 : kNegInf;
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
        st_agent(a.part_m + pb + tid, m_s[tid]);
        st_agent(a.part_l + pb + tid, l_s[tid]);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid + i * 256;
        if (e < R * D) {
            const int r = e / D, d = e - (e / D) * D;
            st_agent(a.part_o + (pb + r) * D + d, acc[i]);
        }
    }
    wait_all_mem();
    __syncthreads();
    if (tid >= 64) return;
    if (!arrive_last(a, bg, tid)) return;
    merge_splits<true, D, 64>(a, bg, b, g, tid);
    if (tid == 0) a.counters[bg] = 0;
}

// --------------------------------------------------------------- host side
AttnPlan attn_plan(int B, int w, int Hq, int Hkv, int D, int tokens, bool f32) {
    AttnPlan p{};
    const int G = Hq / Hkv;
    p.rows = w * G;
    p.rb = (p.rows + 15) / 16;
    if (p.rb == 3) p.rb = 4;   // the bf16 kernel splits its waves over 1, 2 or 4 row blocks
    // head_dim 32: the share fold gives each wave at least 16 columns, so at
    // most two token shares per row block: pad one row block to two
    if (D == 32 && p.rb == 1) p.rb = 2;
    p.rpad = p.rb * 16;
    const long groups = (long)B * Hkv;
    const int tok = tokens > 0 ? tokens : 1;
    // Aim for kAttnTargetGroups work-groups (one 8-wave bf16 group per CU on
    // a 256-CU part).  Every split holds whole tiles (kAttnSplitQuantum tokens
    // covers every tile size of both kernels) and at most kAttnMaxTps tokens.
    // The plan depends on shapes only (not on the dtype), so workspace sizes
    // can be queried without a device.
    (void)f32;
    const long target = kAttnTargetGroups;
    const long quantum = kAttnSplitQuantum;
    long splits = (target + groups - 1) / groups;
    const long max_by_tiles = (tok + quantum - 1) / quantum;
    if (splits > max_by_tiles) splits = max_by_tiles;
    if (splits < 1) splits = 1;
    long tps = (tok + splits - 1) / splits;
    tps = (tps + quantum - 1) / quantum * quantum;
    if (tps > kAttnMaxTps) tps = kAttnMaxTps;
    splits = (tok + tps - 1) / tps;
    p.splits = (int)splits;
    p.tps = (int)tps;
    size_t off = align_up((size_t)kAttnCounterSlots * sizeof(int32_t), 256);
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
    // 8 waves (two per SIMD hide the MFMA / LDS latency of the tile loop)
    // unless a tile would then hold fewer DMA instructions than waves
    // (head_dim 32: a 64-token tile is four DMA instructions per K or V).
    constexpr int NW = (D == 32 || (D == 64 && RB == 4)) ? 4 : (RB == 1 ? 4 : 8);
    const size_t dyn = (size_t)a.tps * sizeof(int);
    if (a.causal) {
        if (a.idx)
            hipLaunchKernelGGL((attn_bf16_kernel<D, RB, NW, false, true>), grid, dim3(NW * 64), dyn, s, a);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<D, RB, NW, true, true>), grid, dim3(NW * 64), dyn, s, a);
    } else {
        if (a.idx)
            hipLaunchKernelGGL((attn_bf16_kernel<D, RB, NW, false, false>), grid, dim3(NW * 64), dyn, s, a);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<D, RB, NW, true, false>), grid, dim3(NW * 64), dyn, s, a);
    }
    return hipGetLastError();
}

#ifdef DUSTIN_ATTN_TRACE
static int g_trace_launches = 0;
#endif

hipError_t launch_attn(const AttnArgs &a_in, const AttnPlan &p, hipStream_t s) {
    AttnArgs a = a_in;
#ifdef DUSTIN_ATTN_TRACE
    a.trace_slot = g_trace_launches++;
#endif
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
            case 3: return launch_bf16<128, 4>(a, grid, s);
            case 4: return launch_bf16<128, 4>(a, grid, s);
        }
    } else if (a.kv.D == 64) {
        switch (p.rb) {
            case 1: return launch_bf16<64, 1>(a, grid, s);
            case 2: return launch_bf16<64, 2>(a, grid, s);
            case 3: return launch_bf16<64, 4>(a, grid, s);
            case 4: return launch_bf16<64, 4>(a, grid, s);
        }
    } else if (a.kv.D == 32) {   // at least two row blocks (attn_plan)
        switch (p.rb) {
            case 2: return launch_bf16<32, 2>(a, grid, s);
            case 4: return launch_bf16<32, 4>(a, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dustin

#ifdef DUSTIN_ATTN_TRACE
// Trace access of the phase-trace build (declared in include/dustin_trace.h).
extern "C" int dustin_trace_attn_read(void *host_dst, size_t bytes) {
    if (bytes < sizeof(dustin::g_attn_trace)) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(dustin::g_attn_trace), sizeof(dustin::g_attn_trace));
}
extern "C" void dustin_trace_attn_restart(void) { dustin::g_trace_launches = 0; }
#endif
