// Fused GQA attention forward, bf16 in / bf16 out, on gfx950 matrix cores.
//
// Method (FlashAttention-2 summary, azimuth.plus): the query rows are cut into
// independent row tiles, one workgroup each (sequence-length parallelism);
// each workgroup streams the K/V tiles of its head once, keeping a running row
// max m, a running sum l and an unnormalised output that is rescaled by
// exp(m_old - m_new) whenever m grows (deferred-normalisation equation for
// O~(j)); the division by l happens once at the end, and the row statistic
// L = m + log(l) is stored. Query rows are spread over the wavefronts of a
// workgroup while all of them share the K/V tile (split-Q). Tiles wholly above
// the causal diagonal are skipped and the element mask is applied only where
// the diagonal or a ragged end crosses a tile.
//
// GQA packing (gitcode GQA guide, PackGQA paragraph; glossary page "How GQA
// works"): a workgroup's 128-row tile holds all G query heads of one K/V head,
// row rho = position * G + head_in_group, so every K/V tile brought on chip is
// used by the whole group. The query-head -> K/V-head map is fixed per
// workgroup before the loop.
//
// gfx950 mapping (our design, not the pages'):
//  * 4 wavefronts x 32 packed rows; v_mfma_f32_32x32x16_bf16 computes the
//    transposed score tile S^T = K Q^T so that each lane owns one query row:
//    the row max and row sum are in-lane plus one v_permlane32_swap.
//  * O^T = V^T P^T accumulates with the same lane <-> query ownership, so the
//    rescale by exp(m_old - m_new) is a per-lane scalar multiply and P never
//    leaves registers (its bf16 copy is the B operand as produced).
//  * K is staged row-major in LDS; V is transposed on its way into LDS.
//    Both are double-buffered, with the next tile's global loads in flight
//    during the current tile's math (one barrier per tile).
//  * exp is 2^x on the transcendental unit with scale*log2(e) folded into one
//    FMA; P and O are rounded to bf16 with round-to-nearest-even.
//  * Workgroup order: head group fastest, so with 8 XCDs and a head-group
//    count divisible by 8 each head group's K/V stays in one XCD's L2; causal
//    row tiles are issued heaviest first.

#include "device_util.h"
#include "params.h"

namespace gqa {

namespace {

constexpr int BM = 128;  // packed query rows per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int NTHREADS = 256;

template <int D>
struct Cfg {
    static constexpr int KS = D + 8;            // LDS row stride of K (elements)
    static constexpr int VS = BN + 4;           // LDS row stride of V^T (elements)
    static constexpr int KQ = D == 128 ? 4 : 2; // keys per thread in the V transpose
    static constexpr int NKL = BN * D / 8 / NTHREADS;  // 16-byte K chunks per thread
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(FwdParams p) {
    constexpr int KS = Cfg<D>::KS, VS = Cfg<D>::VS, KQ = Cfg<D>::KQ, NKL = Cfg<D>::NKL;
    constexpr int DSTEPS = D / 16;  // k-steps of the score product
    constexpr int DBLK = D / 32;    // 32-row blocks of O^T
    constexpr int KB = BN / 32;     // 32-key blocks per tile
    constexpr int C8 = D / 8;       // 16-byte chunks per K/V row

    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * KS];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[2][D * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;

    // ---- workgroup -> (head group, row tile) ----
    const int pid = blockIdx.x;
    const int hg = pid % p.n_hg;
    const int rank = pid / p.n_hg;
    const int rb = CAUSAL ? (p.n_rb - 1 - rank) : rank;
    const int hpb = p.Hq / p.gpack;
    const int b = hg / hpb;
    const int qh0 = (hg - b * hpb) * p.gpack;
    const int kvh = qh0 / p.G;

    int q_tok0, k_tok0, Lq, Lk;
    if (VARLEN) {
        q_tok0 = p.cu_q[b];
        Lq = p.cu_q[b + 1] - q_tok0;
        k_tok0 = p.cu_k[b];
        Lk = p.cu_k[b + 1] - k_tok0;
    } else {
        q_tok0 = b * p.Sq;
        Lq = p.Sq;
        k_tok0 = b * p.Sk;
        Lk = p.Sk;
    }
    const int rows_total = Lq * p.gpack;
    const int row0 = rb * BM;
    if (row0 >= rows_total) return;  // uniform over the workgroup

    const int shift = Lk - Lq;  // bottom-right causal alignment
    int kend = Lk;
    if (CAUSAL) {
        const int last = min(row0 + BM, rows_total) - 1;
        kend = min(Lk, last / p.gpack + 1 + shift);
    }
    const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

    // ---- this lane's query row ----
    const int rho = row0 + wave * 32 + col;
    const bool row_ok = rho < rows_total;
    const int pos = rho / p.gpack;
    const int head = qh0 + (rho - pos * p.gpack);
    const int row_kend = CAUSAL ? min(Lk, pos + 1 + shift) : Lk;

    // ---- this wave's row range: which tiles it needs and which need masking ----
    const int wr0 = row0 + wave * 32;
    const bool wave_live = wr0 < rows_total;
    const int wr1 = min(wr0 + 31, rows_total - 1);
    int wave_kend = Lk, wave_kfull = Lk;
    if (CAUSAL) {
        wave_kend = min(Lk, wr1 / p.gpack + 1 + shift);
        wave_kfull = min(Lk, wr0 / p.gpack + 1 + shift);
    }

    // ---- Q fragment (B operand of S^T = K Q^T), kept in registers ----
    bf16x8 qf[DSTEPS];
    {
        const __bf16 *qrow =
            (const __bf16 *)p.q + ((int64_t)(q_tok0 + pos) * p.Hq + head) * D + 8 * half;
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) {
            if (row_ok) {
                qf[s] = *(const bf16x8 *)(qrow + 16 * s);
            } else {
                qf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
            }
        }
    }

    const int64_t kv_stride = (int64_t)p.Hkv * D;
    const __bf16 *kbase = (const __bf16 *)p.k + ((int64_t)k_tok0 * p.Hkv + kvh) * D;
    const __bf16 *vbase = (const __bf16 *)p.v + ((int64_t)k_tok0 * p.Hkv + kvh) * D;

    // V transpose ownership: keys [va*KQ, va*KQ + KQ) x d [vc*8, vc*8 + 8)
    const int va = tid % (BN / KQ);
    const int vc = tid / (BN / KQ);

    u32x4 kreg[NKL];
    u32x4 vreg[KQ];

    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int c = tid + NTHREADS * i;
            const int r = c / C8, c8 = c % C8;
            const int key = t * BN + r;
            kreg[i] = key < kend ? *(const u32x4 *)(kbase + key * kv_stride + c8 * 8)
                                 : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int qq = 0; qq < KQ; ++qq) {
            const int key = t * BN + va * KQ + qq;
            vreg[qq] = key < kend ? *(const u32x4 *)(vbase + key * kv_stride + vc * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int c = tid + NTHREADS * i;
            const int r = c / C8, c8 = c % C8;
            *(u32x4 *)(&Ks[buf][r * KS + c8 * 8]) = kreg[i];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            __bf16 *lo = &Vt[buf][(vc * 8 + 2 * m) * VS + va * KQ];
            __bf16 *hi = lo + VS;
            if constexpr (KQ == 4) {
                *(u32x2 *)lo = u32x2{pack_lo(vreg[0][m], vreg[1][m]), pack_lo(vreg[2][m], vreg[3][m])};
                *(u32x2 *)hi = u32x2{pack_hi(vreg[0][m], vreg[1][m]), pack_hi(vreg[2][m], vreg[3][m])};
            } else {
                *(uint32_t *)lo = pack_lo(vreg[0][m], vreg[1][m]);
                *(uint32_t *)hi = pack_hi(vreg[0][m], vreg[1][m]);
            }
        }
    };

    const float c = p.scale_log2;
    float m_run = -INFINITY;  // running max of scaled scores, log2 units
    float l_run = 0.f;        // this lane's share of the running sum
    f32x16 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        const bool has_next = t + 1 < ntiles;
        if (has_next) load_tile(t + 1);

        if (wave_live && t * BN < wave_kend) {
            const __bf16 *ks = Ks[cur];
            const __bf16 *vt = Vt[cur];

            // S^T tile: rows = keys, columns = this wave's 32 query rows.
            f32x16 sacc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                sacc[kb] = f32x16{};
                const __bf16 *krow = ks + (kb * 32 + col) * KS + 8 * half;
#pragma unroll
                for (int s = 0; s < DSTEPS; ++s) {
                    const bf16x8 a = *(const bf16x8 *)(krow + 16 * s);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
                }
            }

            // Element mask only on tiles crossing the diagonal or the end.
            if ((t + 1) * BN > wave_kfull) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = t * BN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                        if (key >= row_kend) sacc[kb][r] = -INFINITY;
                    }
            }

            // Online softmax (running max, rescale, exponentials).
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = pair_max32(mx);
            const float m_new = fmaxf(m_run, mx * c);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DBLK; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;

            bf16x8 pf[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float pv = fast_exp2(fmaf(sacc[kb][8 * h2 + j], c, -m_use));
                        l_run += pv;
                        pf[kb][h2][j] = (__bf16)pv;
                    }

            // O^T += V^T P^T. P^T key order in lane (col, half) for k-slot j:
            // key = kb*32 + 16*h2 + 8*(j/4) + 4*half + j%4, matched by the V^T reads.
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int i = 0; i < DBLK; ++i) {
                        const __bf16 *vrow = vt + (i * 32 + col) * VS + kb * 32 + 16 * h2 + 4 * half;
                        const u32x2 lo = *(const u32x2 *)vrow;
                        const u32x2 hi = *(const u32x2 *)(vrow + 8);
                        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                        oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][h2], oacc[i], 0, 0, 0);
                    }
        }

        if (has_next) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: one division by l, L = m + log(l) ----
    const float l_tot = pair_sum32(l_run);
    if (!row_ok) return;
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    __bf16 *orow = (__bf16 *)p.o + ((int64_t)(q_tok0 + pos) * p.Hq + head) * D + 4 * half;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[i][4 * g + e] * inv);
            *(u32x2 *)(orow + i * 32 + 8 * g) = __builtin_bit_cast(u32x2, w);
        }
    if (half == 0) {
        const float lse = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
        const int64_t li = VARLEN ? (int64_t)(q_tok0 + pos) * p.Hq + head
                                  : ((int64_t)b * p.Hq + head) * p.Sq + pos;
        p.lse[li] = lse;
    }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const FwdParams &p, hipStream_t s) {
    const long long grid = (long long)p.n_hg * p.n_rb;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)grid), dim3(NTHREADS), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

int fwd_bf16_rows_per_tile() { return BM; }

hipError_t launch_fwd_bf16(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s) {
#define GQA_CASE(D_, C_, V_) \
    if (d == D_ && causal == C_ && varlen == V_) return launch_t<D_, C_, V_>(p, s);
    GQA_CASE(64, false, false)
    GQA_CASE(64, true, false)
    GQA_CASE(64, false, true)
    GQA_CASE(64, true, true)
    GQA_CASE(128, false, false)
    GQA_CASE(128, true, false)
    GQA_CASE(128, false, true)
    GQA_CASE(128, true, true)
#undef GQA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gqa
