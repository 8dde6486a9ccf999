// Issue probe: does a SIMD's matrix core run while the same SIMD issues plain
// vector (FMA) or transcendental (v_exp_f32) instructions? The forward
// kernels' design depends on the answer. Built as a small program:
//   issue_probe [iterations]  -> one line per case: shader-clock cycles per
//                                iteration per wave, the clock, the SIMD map
//
// Each case runs 256 workgroups (one per CU: 96 KiB of dynamic LDS each) of 4
// or 8 wavefronts. A wavefront's role is its work per iteration:
//   M   8 v_mfma_f32_32x32x16_bf16 on 4 independent accumulators
//   V   64 v_fma_f32 on 16 independent chains
//   E   32 v_exp_f32 on 16 independent chains (x <- 2^-|x|)
//   MV  M and V in one wave, interleaved 1 MFMA : 8 FMA
//   ME  M and E in one wave, interleaved 1 MFMA : 4 exp
//   Mc  8 v_mfma_f32_32x32x16_bf16 accumulating into one accumulator
//   Lb  8 ds_read_b128 (8 KiB per wave, the forward's K operand pattern)
//   Lt  16 ds_read_b64_tr_b16 (8 KiB per wave, the forward's V^T pattern)
//   Lbt both; X both plus the forward's softmax vector work for one tile
//       (16 FMA, 16 exp, 16 add, 8 bf16 packs); L and X roles wait for
//       their LDS reads at the end of each iteration
// With 8 waves, waves w and w + 4 share a SIMD (checked from HW_ID); the first
// role is run by waves 0-3, the second by waves 4-7. Cycles come from
// s_memtime (shader clock) around the loop; the clock from the ratio to
// s_memrealtime (100 MHz). All memory accesses are one store per wave slot of
// the output array, indexed by workgroup and wave.
//
// The compiler keeps MFMA accumulators in AGPRs or in ordinary VGPRs by its
// own heuristic (here: AGPRs, since a wave may use more than 256 registers);
// the program issue_probe_vform is the same source built with
// -mllvm -amdgpu-mfma-vgpr-form, which forces them into VGPRs as in the
// attention kernels (two waves per SIMD, at most 256 registers).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <cstring>

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

enum Role { R_M = 1, R_V = 2, R_E = 3, R_MV = 4, R_ME = 5, R_MC = 6, R_LB = 7, R_LT = 8, R_LBT = 9, R_X = 10 };

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef short s16x4 __attribute__((ext_vector_type(4)));

struct WaveRec {
    unsigned long long cycles, rtc;
    unsigned hwid;
    float sink;
};

__device__ __forceinline__ void loop_m(int iters, f32x16 (&acc)[4], bf16x8 a, bf16x8 b) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[g & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[g & 3], 0, 0, 0);
    }
}

// 8 MFMAs accumulating into one accumulator (a dependent chain)
__device__ __forceinline__ void loop_mc(int iters, f32x16 (&acc)[4], bf16x8 a, bf16x8 b) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[0], 0, 0, 0);
    }
}

// LDS reads in the forward kernel's d = 128 operand patterns, 8 KiB per
// wave each: 8 ds_read_b128 (a 32 x 128 bf16 K tile) and 16
// ds_read_b64_tr_b16 (the transposed V tile). The values are kept alive by
// empty asm statements; each iteration waits for its reads.
struct LdsAddr {
    uint32_t kb[8];  // byte offsets of the b128 reads
    uint32_t vt[4];  // byte offsets of the transposing reads (+ 2048 / 4096 / 6144 for the others)
};
__device__ __forceinline__ LdsAddr lds_addr_of(int lane) {
    LdsAddr a;
    const int col = lane & 31, half = lane >> 5;
    for (int s = 0; s < 8; ++s) a.kb[s] = (col * 128 + (((2 * s + half) ^ (col & 15)) * 8)) * 2;
    const int vj = lane & 15, vg = lane >> 4;
    const int v_row = 4 * (vg >> 1) + (vj >> 2);
    for (int i = 0; i < 4; ++i) {
        const int chunk = 4 * i + 2 * (vg & 1) + ((vj & 3) >> 1);
        a.vt[i] = 16384 + (v_row * 128 + ((chunk ^ (4 * (v_row & 3))) * 8) + 4 * (vj & 1)) * 2;
    }
    return a;
}
__device__ __forceinline__ void lds_reads(const unsigned char *lds, const LdsAddr &a, bool b128, bool tr) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    // every read is issued before any value is consumed (distinct
    // destination registers), so the reads pipeline as they do in the
    // kernels, and the caller's wait at the end of the iteration measures
    // their throughput rather than one latency per read
    u32x4 kv[8];
    s16x4 tv[16];
    if (b128) {
#pragma unroll
        for (int s = 0; s < 8; ++s) kv[s] = *(const u32x4 *)(lds + a.kb[s]);
    }
    if (tr) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tv[4 * h + i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds + a.vt[i] + 2048 * h));
    }
    if (b128) {
#pragma unroll
        for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(kv[s]));
    }
    if (tr) {
#pragma unroll
        for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(tv[j]));
    }
}
__device__ __forceinline__ void loop_l(int iters, const unsigned char *lds, const LdsAddr &a, bool b128, bool tr) {
    for (int i = 0; i < iters; ++i) {
        lds_reads(lds, a, b128, tr);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}
// The forward step's softmax cluster: 16 x (FMA, exp, add), 8 bf16 packs,
// with both LDS read patterns.
__device__ __forceinline__ void loop_x(int iters, const unsigned char *lds, const LdsAddr &a, float (&x)[16],
                                       float fa, float fb) {
    for (int i = 0; i < iters; ++i) {
        lds_reads(lds, a, true, true);
        float part[4] = {0.f, 0.f, 0.f, 0.f};
        uint32_t pk[8];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(x[j], fa, -fb));
            part[j & 3] += p;
            x[j] = p;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            const bf2 v = {(__bf16)x[2 * j], (__bf16)x[2 * j + 1]};
            pk[j] = __builtin_bit_cast(uint32_t, v);
            asm volatile("" ::"v"(pk[j]));
        }
        x[0] += (part[0] + part[1]) + (part[2] + part[3]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

__device__ __forceinline__ void loop_v(int iters, float (&x)[16], float fa, float fb) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int g = 0; g < 64; ++g) x[g & 15] = fmaf(x[g & 15], fa, fb);
    }
}

__device__ __forceinline__ void loop_e(int iters, float (&x)[16]) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int g = 0; g < 32; ++g) x[g & 15] = __builtin_amdgcn_exp2f(-fabsf(x[g & 15]));
    }
}

__device__ __forceinline__ void loop_mv(int iters, f32x16 (&acc)[4], bf16x8 a, bf16x8 b, float (&x)[16],
                                        float fa, float fb) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            acc[g & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[g & 3], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) x[(8 * g + j) & 15] = fmaf(x[(8 * g + j) & 15], fa, fb);
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
    }
}

__device__ __forceinline__ void loop_me(int iters, f32x16 (&acc)[4], bf16x8 a, bf16x8 b, float (&x)[16]) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            acc[g & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[g & 3], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[(4 * g + j) & 15] = __builtin_amdgcn_exp2f(-fabsf(x[(4 * g + j) & 15]));
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
    }
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void probe_kernel(WaveRec *out, int iters, int role_lo, int role_hi,
                                                        float fa, float fb) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_dyn[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave < 4 ? role_lo : role_hi;
    const LdsAddr la = lds_addr_of(lane);
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(0.001f * (lane + j));
        b[j] = (__bf16)(0.002f * (lane - j));
    }
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 0.01f * (lane + j);

    __syncthreads();
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    if (role == R_M) loop_m(iters, acc, a, b);
    else if (role == R_V) loop_v(iters, x, fa, fb);
    else if (role == R_E) loop_e(iters, x);
    else if (role == R_MV) loop_mv(iters, acc, a, b, x, fa, fb);
    else if (role == R_ME) loop_me(iters, acc, a, b, x);
    else if (role == R_MC) loop_mc(iters, acc, a, b);
    else if (role == R_LB) loop_l(iters, lds_dyn, la, true, false);
    else if (role == R_LT) loop_l(iters, lds_dyn, la, false, true);
    else if (role == R_LBT) loop_l(iters, lds_dyn, la, true, true);
    else if (role == R_X) loop_x(iters, lds_dyn, la, x, fa, fb);
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
    if (lane == 0) {
        WaveRec rec;
        rec.cycles = c1 - c0;
        rec.rtc = r1 - r0;
        rec.hwid = __builtin_amdgcn_s_getreg((31 << 11) | 4);  // HW_ID, bits 31:0
        rec.sink = s;
        out[blockIdx.x * NW + wave] = rec;
    }
}

static const char *role_name(int r) {
    switch (r) {
    case R_M: return "M";
    case R_V: return "V";
    case R_E: return "E";
    case R_MV: return "MV";
    case R_ME: return "ME";
    case R_MC: return "Mc";
    case R_LB: return "Lb";
    case R_LT: return "Lt";
    case R_LBT: return "Lbt";
    case R_X: return "X";
    default: return "-";
    }
}

int main(int argc, char **argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 2000;
    const int grid = 256;
    WaveRec *d_out;
    if (hipMalloc(&d_out, sizeof(WaveRec) * grid * 8) != hipSuccess) {
        printf("alloc failed\n");
        return 1;
    }
    WaveRec h[256 * 8];
    struct Case { int nw, lo, hi; };
    const Case cases[] = {
        {4, R_M, R_M},   {4, R_V, R_V},   {4, R_E, R_E},   {4, R_MV, R_MV}, {4, R_ME, R_ME},
        {8, R_M, R_M},   {8, R_V, R_V},   {8, R_E, R_E},   {8, R_M, R_V},   {8, R_M, R_E},
        {8, R_MV, R_MV}, {8, R_ME, R_ME}, {4, R_MC, R_MC}, {8, R_MC, R_V}, {8, R_MC, R_E},
        {4, R_LB, R_LB}, {4, R_LT, R_LT}, {4, R_LBT, R_LBT}, {8, R_LBT, R_LBT}, {8, R_M, R_LBT},
        {4, R_X, R_X},   {8, R_M, R_X},   {8, R_X, R_X},
    };
    const size_t lds = 96 * 1024;  // one workgroup per CU
    if (hipFuncSetAttribute((const void *)probe_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
            hipSuccess ||
        hipFuncSetAttribute((const void *)probe_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
            hipSuccess) {
        printf("attribute failed\n");
        return 1;
    }
    for (int rep = 0; rep < 2; ++rep) {  // the first pass warms the clocks up
        for (const Case &c : cases) {
            if (c.nw == 4)
                hipLaunchKernelGGL(probe_kernel<4>, dim3(grid), dim3(256), lds, 0, d_out, iters, c.lo, c.hi,
                                   0.999f, 0.001f);
            else
                hipLaunchKernelGGL(probe_kernel<8>, dim3(grid), dim3(512), lds, 0, d_out, iters, c.lo, c.hi,
                                   0.999f, 0.001f);
            if (hipDeviceSynchronize() != hipSuccess) {
                printf("launch failed\n");
                return 1;
            }
            if (rep == 0) continue;
            hipMemcpy(h, d_out, sizeof(WaveRec) * grid * c.nw, hipMemcpyDeviceToHost);
            double cyc[2] = {0, 0}, rtc = 0;
            int n[2] = {0, 0}, same_simd = 0;
            for (int g = 0; g < grid; ++g) {
                for (int w = 0; w < c.nw; ++w) {
                    const WaveRec &r = h[g * c.nw + w];
                    cyc[w >= 4] += (double)r.cycles;
                    n[w >= 4]++;
                    rtc += (double)r.rtc;
                    if (c.nw == 8 && w < 4) {
                        const unsigned s0 = (r.hwid >> 4) & 3, s1 = (h[g * 8 + w + 4].hwid >> 4) & 3;
                        same_simd += s0 == s1;
                    }
                }
            }
            const double ghz = (cyc[0] + cyc[1]) / rtc * 0.1;
            printf("waves/SIMD %d  roles %-2s | %-2s  cycles/iter %7.1f | %7.1f  clock %.2f GHz", c.nw / 4,
                   role_name(c.lo), c.nw == 8 ? role_name(c.hi) : "-", cyc[0] / n[0] / iters,
                   n[1] ? cyc[1] / n[1] / iters : 0.0, ghz);
            if (c.nw == 8) printf("  pairs on one SIMD %d/%d", same_simd, grid * 4);
            printf("\n");
        }
    }
    hipFree(d_out);
    return 0;
}
