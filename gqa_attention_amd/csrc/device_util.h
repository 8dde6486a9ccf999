// Small device helpers for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef uint32_t u32x8_t __attribute__((__vector_size__(8 * sizeof(uint32_t))));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Largest amount (log2 units) by which a tile's row max may exceed the running
// reference max before the unnormalised output is rescaled (p <= 2^8 = 256).
constexpr float kRescaleGap = 8.0f;
// Largest sum of one lane's probabilities over a forward tile (16 values)
// before the tile is recomputed against a raised reference max; every p of an
// accepted tile is then <= 2^12.
constexpr float kTileSumBound = 4096.0f;

// Combine a value with the one held by lane (l ^ 32). v_permlane32_swap
// exchanges the two 32-lane halves, so (r[0], r[1]) hold the pair
// {x[l % 32], x[l % 32 + 32]} in every lane; a symmetric op on them is the
// same, bit for bit, in both lanes of a pair.
__device__ __forceinline__ float pair_max32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane j supplies the address of 4 consecutive 16-bit elements; viewing the
// group's 64 elements as E[4j + e], lane c receives E[c], E[c+16], E[c+32],
// E[c+48]. With lane j pointing at row (j / 4), columns 4 (j % 4) .. +3 of a
// row-major tile, lane c gets the 4 rows of column c: a column slice of V as
// the matrix-core operand of V^T.
typedef short s16x4_lds __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16 *p) {
    const s16x4_lds t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_lds *)(p));
    return __builtin_bit_cast(u32x2, t);
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds_base + 16 l, lds_base being
// wave-uniform (M0). Written as asm so that the compiler does not track it:
// callers wait for completion themselves with s_waitcnt vmcnt. It has no
// register outputs; its inputs are read when it issues. The compiler's own
// vmcnt waits do not count these loads and can therefore only over-wait.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; nothing else here uses it
__device__ __forceinline__ void lds_dma16(const void *gptr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}
// The same for an LDS address the compiler may hold in a vector register
// (it must still be the same in every lane): readfirstlane moves it to an
// SGPR for M0.
__device__ __forceinline__ void lds_dma16_u(const void *gptr, uint32_t lds_base) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m), "v"(gptr)
                 : "memory", "m0");
}
// The same load addressed as a wave-uniform 64-bit base (scalar registers)
// plus a 32-bit per-lane byte offset: the next tile is reached by scalar
// arithmetic and the per-lane offsets of a full tile stay fixed.
__device__ __forceinline__ void lds_dma16_sv(const void *sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
// A wave-uniform pointer the compiler may hold in vector registers (a loop
// induction variable, say), read from the first lane into scalar registers.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return (const void *)(uintptr_t)(lo | hi << 32);
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 2^x on the transcendental unit (v_exp_f32); exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Longest first over the sequences of a packed batch (prefix offsets cu_q,
// cu_k, B <= kLptMax <= threads per workgroup): returns the index of the
// sequence whose work Lq x Lk ranks r-th largest (ties by index). Workgroups
// start roughly in blockIdx order, so giving rank r to the r-th group of
// workgroups starts the heaviest pieces first. Every thread of the workgroup
// must call it (two barriers).
constexpr int kLptMax = 64;
__device__ __forceinline__ int lpt_sequence(const int32_t *cu_q, const int32_t *cu_k, int B, int r,
                                            int tid) {
    __shared__ long long s_work[kLptMax];
    __shared__ int s_pick;
    if (tid < B) s_work[tid] = (long long)(cu_q[tid + 1] - cu_q[tid]) * (cu_k[tid + 1] - cu_k[tid]);
    __syncthreads();
    if (tid < B) {
        const long long mine = s_work[tid];
        int rank = 0;
        for (int y = 0; y < B; ++y) {
            const long long o = s_work[y];
            rank += (o > mine) || (o == mine && y < tid);
        }
        if (rank == r) s_pick = tid;
    }
    __syncthreads();
    return s_pick;
}

// fp8 e4m3 -> bf16 (exact: every e4m3 value is a bf16 value) for 4 packed
// values.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Pack the low / high bf16 halves of two dwords: (lo(a), lo(b)) and (hi(a), hi(b)).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}

}  // namespace gqa
