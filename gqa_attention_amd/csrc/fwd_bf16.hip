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
//  * K and V are staged row-major in LDS (coalesced 16-byte loads of whole
//    rows); the V^T operand is read with ds_read_b64_tr_b16, which hands each
//    lane a column slice. Double-buffered, with the next tile's global loads
//    in flight during the current tile's math (one barrier per tile).
//  * exp is 2^x on the transcendental unit with scale*log2(e) folded into one
//    FMA; P and O are rounded to bf16 with round-to-nearest-even.
//  * Workgroup order: the row tiles of a head group run back to back on one
//    XCD (workgroups are dealt round-robin to the 8 XCDs), so its K/V comes
//    from HBM once and is then reused from that XCD's L2; causal row tiles are
//    issued heaviest first.

#include "device_util.h"
#include "params.h"

namespace gqa {

namespace {

constexpr int BM = 128;  // packed query rows per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int NTHREADS = 256;

template <int D>
struct Cfg {
    static constexpr int KS = D + 8;    // LDS row stride of K (elements): conflict-free b128 reads
    static constexpr int VS = D + 32;   // LDS row stride of V (elements): conflict-free tr16 reads
    static constexpr int NKL = BN * D / 8 / NTHREADS;  // 16-byte chunks per thread per tensor
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(FwdParams p) {
    constexpr int KS = Cfg<D>::KS, VS = Cfg<D>::VS, NKL = Cfg<D>::NKL;
    constexpr int DSTEPS = D / 16;  // k-steps of the score product
    constexpr int DBLK = D / 32;    // 32-row blocks of O^T
    constexpr int KB = BN / 32;     // 32-key blocks per tile
    constexpr int C8 = D / 8;       // 16-byte chunks per K/V row

    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * KS];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BN * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;

    // ---- workgroup -> (head group, row tile) ----
    // Workgroups are dealt round-robin to the 8 XCDs (pid % 8). When the head
    // groups split evenly over the XCDs, all row tiles of one head group run
    // back to back on one XCD, so its K/V is fetched from HBM once and then
    // served from that XCD's L2. Causal row tiles go heaviest first.
    const int pid = blockIdx.x;
    int hg, rank;
    if ((p.n_hg & 7) == 0) {
        const int slot = pid >> 3;
        hg = (slot / p.n_rb) * 8 + (pid & 7);
        rank = slot % p.n_rb;
    } else {
        hg = pid / p.n_rb;
        rank = pid % p.n_rb;
    }
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

    // Tile staging: thread tid moves 16-byte chunks tid + 256 i (row-major,
    // D/8 chunks per row) of K and of V. Offsets are fixed per thread.
    int g_off[NKL], k_soff[NKL], v_soff[NKL], row_of[NKL];
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
        const int c = tid + NTHREADS * i;
        row_of[i] = c / C8;
        g_off[i] = (c % C8) * 8;
        k_soff[i] = row_of[i] * KS + g_off[i];
        v_soff[i] = row_of[i] * VS + g_off[i];
    }
    u32x4 kreg[NKL], vreg[NKL];

    // Rows past kend are clamped to the last needed key: they are real, finite
    // K/V rows, their scores are masked to -inf and their p is exactly 0.
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int64_t off = (int64_t)min(t * BN + row_of[i], kend - 1) * kv_stride + g_off[i];
            kreg[i] = *(const u32x4 *)(kbase + off);
            vreg[i] = *(const u32x4 *)(vbase + off);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            *(u32x4 *)(&Ks[buf][k_soff[i]]) = kreg[i];
            *(u32x4 *)(&Vs[buf][v_soff[i]]) = vreg[i];
        }
    };

    // V^T operand through ds_read_b64_tr_b16: in 16-lane group g, lane j reads
    // row key0 + j/4, columns d0 + 4 (j%4) .. +3 and receives column d0 + j of
    // rows key0 .. key0+3, with d0 = 32 i + 16 (g & 1) and key0 = 4 (g >> 1)
    // (+ 8 for the second read) inside the 16-key slot.
    const int vj = lane & 15, vg = lane >> 4;
    const int v_rd = (4 * (vg >> 1) + (vj >> 2)) * VS + 16 * (vg & 1) + 4 * (vj & 3);
    const int k_rd = col * KS + 8 * half;

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
            const __bf16 *vs = Vs[cur];

            // S^T tile: rows = keys, columns = this wave's 32 query rows.
            f32x16 sacc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                sacc[kb] = f32x16{};
                const __bf16 *krow = ks + kb * 32 * KS + k_rd;
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
            // The reference max only moves when the tile max exceeds it by more
            // than kRescaleGap (log2 units); every p then stays <= 2^kRescaleGap
            // and the rescale of O~ is skipped on almost every tile. The result
            // is the same: m cancels between O~ and l and is added back in L.
            const float mxs = mx * c;
            if (mxs > m_run + kRescaleGap) {
                const float alpha = fast_exp2(m_run - mxs);
                m_run = mxs;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < DBLK; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;

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
                        const __bf16 *vp = vs + (kb * 32 + 16 * h2) * VS + 32 * i + v_rd;
                        const u32x2 lo = lds_read_tr16(vp);
                        const u32x2 hi = lds_read_tr16(vp + 8 * VS);
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
