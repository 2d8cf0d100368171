// Device-side helpers shared by the gfx950 kernels of the sparse-verification
// step: vector types for the MFMA operands, bf16 conversion, wave64
// reductions and the LDS-DMA / waitcnt wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dustin {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kFltMax = 3.40282347e+38f;   // largest finite float

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t x = __float_as_uint(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((x >> 16) | 0x40u);
    x += 0x7fffu + ((x >> 16) & 1u);
    return static_cast<uint16_t>(x >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Reduce across the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48).
// (v_permlane32_swap / v_permlane16_swap would avoid the LDS round trip of
// these shuffles, but made the attention output depend on timing in one
// 4-wave configuration; the shuffles are deterministic.)
__device__ __forceinline__ float group4_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float group4_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

// Reduce across the 16 lanes of one 16-lane group (a DPP row): rotations
// by 8, 4, 2 and 1 within the row leave the full result in every lane,
// with register-only DPP moves rather than LDS shuffles.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane16_sum(float v) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    return v + row_ror<1>(v);
}
__device__ __forceinline__ float lane16_max(float v) {
    v = fmaxf(v, row_ror<8>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<2>(v));
    return fmaxf(v, row_ror<1>(v));
}

// 16-byte streaming load (nontemporal: the data is read once per pass and
// should not displace cached data).  Only for accesses whose instruction
// covers whole cache lines: a line split over two instructions is then
// fetched twice.
__device__ __forceinline__ u32x4 ld_stream16(const void *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// Asynchronous 16-byte-per-lane copy global -> LDS.  `lds_base` is the
// wave-uniform destination; lane i lands at lds_base + 16 * i.
__device__ __forceinline__ void dma16(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (lds_void_t *)lds_base, 16, 0, 0);
}
// The same with the nontemporal cache policy, for rows read once per call:
// the gathered K/V rows (every instruction covers whole 128-byte lines).
// Measured ~9% faster per attention launch than the default policy.
constexpr int kCachePolicyNt = 2;
__device__ __forceinline__ void dma16_stream(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (lds_void_t *)lds_base, 16, 0, kCachePolicyNt);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Work-group barrier for hand-offs through LDS only.  __syncthreads() also
// fences global memory, and on gfx950 that makes every wave wait for all of
// its outstanding vector-memory operations, including global->LDS DMA issued
// for later pipeline stages, at every barrier.  This barrier waits only for
// the wave's own LDS accesses (lgkmcnt(0)); callers first wait, with
// wait_vmcnt, for exactly the DMA the next stage reads.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Device-coherent ("agent scope") relaxed loads and stores.  On gfx950 they
// are issued with the sc1 cache policy: stores write through the XCD-local
// L2 and loads do not hit stale L2 lines, so data exchanged between
// work-groups on different XCDs needs no L2 write-back or invalidation.
__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent4(float *p, f32x4 v) {
    st_agent(p, v[0]);
    st_agent(p + 1, v[1]);
    st_agent(p + 2, v[2]);
    st_agent(p + 3, v[3]);
}
__device__ __forceinline__ f32x4 ld_agent4(const float *p) {
    return f32x4{ld_agent(p), ld_agent(p + 1), ld_agent(p + 2), ld_agent(p + 3)};
}
// Device-coherent loads through a buffer resource: buffer_load with the sc1
// cache policy reads the coherent copy (no stale XCD-local L2 line) while the
// compiler schedules and overlaps them like ordinary loads.  Loads past
// `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ float ld_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCachePolicySc1));
}
__device__ __forceinline__ f32x4 ld_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCachePolicySc1));
}
// 16-byte device-coherent store: buffer_store_dwordx4 with the sc1 cache
// policy writes through the XCD-local L2.  (A compiler builtin rather than
// inline assembly: the compiler must see the store to keep its data
// registers intact until the store has read them.)
__device__ __forceinline__ void st_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kCachePolicySc1);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// LDS byte address (the offset register value of ds_* instructions).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(lds_void_t *)p;
}

// 32-bit LDS reads that have completed when they return.  Inline assembly:
// the compiler cannot always tell a C++ read of LDS apart from the target of
// a pending global->LDS DMA, and then puts a wait for every outstanding
// vector-memory request in front of it, which empties a streaming ring.
__device__ __forceinline__ int lds_read_i32(const void *p) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
    return v;
}
__device__ __forceinline__ float lds_read_f32(const void *p) {
    float v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
    return v;
}

// Transposed LDS reads (ds_read_b64_tr_b16) of the V operand of the PV
// product, issued as one block that also waits for their completion.  Within
// each 16-lane group, lane i receives element (i mod 4) of the 8-byte rows
// addressed by lanes 4t + i/4, t = 0..3.  addr[d] is this lane's address for
// the first row quad of d tile d; the second quad sits OFF1 bytes further.
// Written as inline assembly so that the compiler does not serialise these
// reads behind the global->LDS copies still in flight to other buffers.
template <int OFF1>
__device__ __forceinline__ void ds_read_tr16_x8(const uint32_t (&addr)[8], s16x4 (&lo)[8], s16x4 (&hi)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:%c24\n\t"
        "ds_read_b64_tr_b16 %2, %17\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:%c24\n\t"
        "ds_read_b64_tr_b16 %4, %18\n\t"
        "ds_read_b64_tr_b16 %5, %18 offset:%c24\n\t"
        "ds_read_b64_tr_b16 %6, %19\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%c24\n\t"
        "ds_read_b64_tr_b16 %8, %20\n\t"
        "ds_read_b64_tr_b16 %9, %20 offset:%c24\n\t"
        "ds_read_b64_tr_b16 %10, %21\n\t"
        "ds_read_b64_tr_b16 %11, %21 offset:%c24\n\t"
        "ds_read_b64_tr_b16 %12, %22\n\t"
        "ds_read_b64_tr_b16 %13, %22 offset:%c24\n\t"
        "ds_read_b64_tr_b16 %14, %23\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%c24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
          "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5]),
          "=&v"(lo[6]), "=&v"(hi[6]), "=&v"(lo[7]), "=&v"(hi[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]),
          "v"(addr[6]), "v"(addr[7]), "i"(OFF1)
        : "memory");
}

template <int OFF1>
__device__ __forceinline__ void ds_read_tr16_x2(const uint32_t (&addr)[2], s16x4 (&lo)[2], s16x4 (&hi)[2]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%c6\n\t"
        "ds_read_b64_tr_b16 %2, %5\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%c6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
        : "v"(addr[0]), "v"(addr[1]), "i"(OFF1)
        : "memory");
}

template <int OFF1>
__device__ __forceinline__ void ds_read_tr16_x1(const uint32_t (&addr)[1], s16x4 (&lo)[1], s16x4 (&hi)[1]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:%c3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0])
        : "v"(addr[0]), "i"(OFF1)
        : "memory");
}

template <int OFF1>
__device__ __forceinline__ void ds_read_tr16_x4(const uint32_t (&addr)[4], s16x4 (&lo)[4], s16x4 (&hi)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%c12\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%c12\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%c12\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%c12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
          "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(OFF1)
        : "memory");
}

// N single transposed reads (one per d tile, 4 tokens each) plus their
// completion wait, for the 16x16x16 PV product.
__device__ __forceinline__ void ds_read_tr16_n8(const uint32_t (&a)[8], s16x4 (&v)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}
__device__ __forceinline__ void ds_read_tr16_n4(const uint32_t (&a)[4], s16x4 (&v)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}
// N x ds_read_b128 as inline asm.  The compiler treats any C++ read of an LDS
// buffer that global->LDS DMA writes as possibly aliasing DMA still in
// flight and waits for all outstanding vector-memory operations first; the
// pipelined kernels order these reads themselves (wait_vmcnt + lds_barrier).
__device__ __forceinline__ void ds_read_b128_n(const uint32_t (&a)[4], u32x4 (&v)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}
__device__ __forceinline__ void ds_read_b128_n(const uint32_t (&a)[1], u32x4 (&v)[1]) {
    asm volatile(
        "ds_read_b128 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0])
        : "v"(a[0])
        : "memory");
}
__device__ __forceinline__ void ds_read_b128_n(const uint32_t (&a)[2], u32x4 (&v)[2]) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(a[0]), "v"(a[1])
        : "memory");
}

__device__ __forceinline__ void ds_read_tr16_n2(const uint32_t (&a)[2], s16x4 (&v)[2]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(a[0]), "v"(a[1])
        : "memory");
}

template <int N>
__device__ __forceinline__ void ds_read_tr16_n(const uint32_t (&a)[N], s16x4 (&v)[N]) {
    static_assert(N == 8 || N == 4 || N == 2, "d tiles");
    if constexpr (N == 8) ds_read_tr16_n8(a, v);
    else if constexpr (N == 4) ds_read_tr16_n4(a, v);
    else ds_read_tr16_n2(a, v);
}

// Dispatch on the number of d tiles.
template <int N, int OFF1>
__device__ __forceinline__ void ds_read_tr16(const uint32_t (&addr)[N], s16x4 (&lo)[N], s16x4 (&hi)[N]) {
    if constexpr (N == 8) ds_read_tr16_x8<OFF1>(addr, lo, hi);
    else if constexpr (N == 4) ds_read_tr16_x4<OFF1>(addr, lo, hi);
    else if constexpr (N == 2) ds_read_tr16_x2<OFF1>(addr, lo, hi);
    else ds_read_tr16_x1<OFF1>(addr, lo, hi);
}

}  // namespace dustin
