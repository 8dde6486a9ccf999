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
// With 8 waves, waves w and w + 4 share a SIMD (checked from HW_ID); the first
// role is run by waves 0-3, the second by waves 4-7. Cycles come from
// s_memtime (shader clock) around the loop; the clock from the ratio to
// s_memrealtime (100 MHz). All memory accesses are one store per wave slot of
// the output array, indexed by workgroup and wave.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

enum Role { R_M = 1, R_V = 2, R_E = 3, R_MV = 4, R_ME = 5 };

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
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave < 4 ? role_lo : role_hi;
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
        {8, R_MV, R_MV}, {8, R_ME, R_ME},
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
