// Split-KV GQA decode (bf16) and the log-sum-exp combine of split partials.
//
// Decode: one new query token per sequence reads its whole K/V cache, so the
// step is bound by HBM bandwidth (Ultralytics glossary, "How GQA shrinks the
// KV cache"). The cache's key range is cut into num_splits contiguous ranges
// (gitcode GQA guide, num_splits); each range gives a normalised partial
// output O_s and its log-sum-exp L_s, and the partials are merged exactly
// through L = M + log sum_s exp(L_s - M), O = sum_s exp(L_s - L) O_s (the
// pages print no merge; this follows from the LSE definition on the
// FlashAttention-2 page, L = m + log l).
//
// gfx950 mapping (our design):
//  * workgroup = (batch, K/V head, split, slice of up to 16 query heads of
//    the group): every K/V byte of the range is read from HBM exactly once
//    and used by all G heads of the group (pack_gqa).
//  * 4 wavefronts per workgroup, each streaming its own 32-key tiles (tiles
//    w, w+4, ...) with its own running max / sum; the 4 partial states are
//    merged through LDS at the end.
//  * v_mfma_f32_16x16x32_bf16 for S^T = K Q^T (16 keys x 16 query heads) with
//    K loaded from HBM straight into the A-operand layout, and for
//    O^T = V^T P^T with V staged row-major in a wave-private LDS slice and
//    read as V^T with ds_read_b64_tr_b16. The next tile's loads are issued
//    before the current tile's math.

#include <type_traits>

#include "device_util.h"
#include "params.h"

namespace gqa {

namespace {

#ifndef GQA_DEC_WPE
#define GQA_DEC_WPE 2  // waves per SIMD the register budget is sized for
#endif

// K/V cache loads. Every cache byte is read once per call. V rows (whole
// 16-byte chunks of each row, 16 lanes per bf16 row) carry the non-temporal
// hint; K loads keep the default policy. Measured on B 64 x 4096 keys, 32/8
// heads, d 128 against the hint on both: ns 1 / 2 / 4 / 8 at 6.31 / 6.04 /
// 5.96 / 6.07 TB/s instead of 5.85 / 5.66 / 5.64 / 5.65; on the ragged paged
// fp8 cache the hint on V alone gives +11-13 % over no hint and the hint on
// K costs 4 %.
template <typename T, bool NT>
__device__ __forceinline__ T load_kv(const unsigned char *ptr) {
    if constexpr (NT)
        return __builtin_nontemporal_load((const T *)ptr);
    else
        return *(const T *)ptr;
}

constexpr int NTHREADS = 256;
constexpr int NWAVES = 4;
constexpr int TK = 32;        // keys per wave tile

template <int D>
struct DecCfg {
    static constexpr int NS = D / 32;    // k-steps of 32 head_dim elements
    static constexpr int NDT = D / 16;   // 16-row tiles of O^T
    static constexpr int NVL = D / 16;   // 16-byte bf16 V chunks per lane per tile
    // V row stride in LDS (elements): the 32 lanes of a transposing read touch
    // rows r..r+3 and r+4..r+7; a stride of D + 16 puts their 8 segments of
    // 32 bytes on disjoint banks.
    static constexpr int VRS = D + 16;
    static constexpr int VT_BYTES = NWAVES * TK * VRS * 2;
    static constexpr int MERGE_BYTES = (NWAVES * D * 16 + 2 * NWAVES * 16) * 4;
    static constexpr int SMEM = VT_BYTES > MERGE_BYTES ? VT_BYTES : MERGE_BYTES;
};
// Block-table entries staged in LDS at a time (paged caches); a split that
// spans more blocks is walked in windows of this many blocks.
constexpr int MAX_TBL = 2048;
// Ragged batches of at most this many sequences are scheduled longest first.
constexpr int LPT_MAX = 256;
static_assert(LPT_MAX <= NTHREADS, "one thread ranks one sequence");

template <int D, bool PAGED, bool FP8>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(GQA_DEC_WPE))) void
decode_bf16_kernel(DecodeParams p) {
    constexpr int NS = DecCfg<D>::NS, NDT = DecCfg<D>::NDT;
    constexpr int VRS = DecCfg<D>::VRS;
    constexpr int ESZ = FP8 ? 1 : 2;                // bytes per cached element
    constexpr int VCH = 16 / ESZ;                   // elements per 16-byte V load
    constexpr int VCPR = D / VCH;                   // V loads per row
    constexpr int NVL = TK * VCPR / 64;             // V loads per lane per tile
    typedef typename std::conditional<FP8, u32x2, bf16x8>::type kraw_t;  // K operand as loaded
    __shared__ __attribute__((aligned(16))) unsigned char smem[DecCfg<D>::SMEM];
    __shared__ int tbl[PAGED ? MAX_TBL : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int qi = lane & 15, kq = lane >> 4;

    // blockIdx.x -> (query slice, split, K/V head, sequence rank); slices fastest.
    int id = blockIdx.x;
    const int qs = id % p.n_qs;
    id /= p.n_qs;
    const int split = id % p.num_splits;
    id /= p.num_splits;
    const int kvh = id % p.Hkv;
    const int rank = id / p.Hkv;

    const int qg = qs * 16 + qi;  // head within the group
    const bool q_ok = qg < p.G;
    const int head = kvh * p.G + qg;

    // Keys of sequence x visible to its new token: [vis_lo, L), the last
    // window_left + 1 keys with a sliding window.
    auto seq_len = [&](int x) { return p.seqlens ? min(max(p.seqlens[x], 0), p.Sk) : p.Sk; };
    auto first_visible = [&](int L) {
        return p.window_left >= 0 ? max(0, L - 1 - p.window_left) : 0;
    };

    // Longest first: workgroups start roughly in blockIdx order, so with
    // per-sequence lengths the sequence of rank r (r-th longest visible
    // range, ties by index) gets the r-th group of workgroups. The biggest
    // pieces start first and the short ones fill the tail.
    int b = rank;
    if (p.seqlens && p.B > 1 && p.B <= LPT_MAX) {
        __shared__ int s_pick;
        int *vis = (int *)smem;  // [B] visible lengths (smem holds V tiles later)
        for (int x = tid; x < p.B; x += NTHREADS) {
            const int Lx = seq_len(x);
            vis[x] = Lx - first_visible(Lx);
        }
        __syncthreads();
        if (tid < p.B) {
            const int mine = vis[tid];
            int r = 0;
            for (int y = 0; y < p.B; ++y) {
                const int o = vis[y];
                r += (o > mine) || (o == mine && y < tid);
            }
            if (r == rank) s_pick = tid;
        }
        __syncthreads();
        b = s_pick;
    }

    // This sequence's visible keys, cut into num_splits contiguous ranges of
    // ceil(n / num_splits) keys rounded up to a multiple of 64.
    const int L = seq_len(b);
    const int vis_lo = first_visible(L);
    const int n = L - vis_lo;
    const int chunk = (int)((((int64_t)n + p.num_splits - 1) / p.num_splits + 63) & ~(int64_t)63);
    const int k_lo = vis_lo + (int)min((int64_t)n, (int64_t)split * chunk);
    const int k_hi = vis_lo + (int)min((int64_t)n, (int64_t)(split + 1) * chunk);
    const int rows = p.B * p.Hq;
    if (p.num_splits > 1 && k_hi <= k_lo) {
        // A split past the sequence's end: the merge only needs its LSE (-inf).
        if (tid < 16 && qs * 16 + tid < p.G)
            p.ws_lse[(int64_t)split * rows + (int64_t)b * p.Hq + kvh * p.G + qs * 16 + tid] = -INFINITY;
        return;
    }

    // Q^T fragment (B operand): head_dim elements 32*s + 8*kq + j of query qi.
    bf16x8 qf[NS];
    {
        // k-step s of lane group kq holds head_dim elements 8 kq + 32 s .. +7
        // (bf16 cache) or 8 NS kq + 8 s .. +7 (fp8 cache, so that a lane's K
        // codes for all steps are one contiguous run); K follows the same map.
        const __bf16 *qrow = (const __bf16 *)p.q + ((int64_t)b * p.Hq + head) * D +
                             (FP8 ? 8 * NS * kq : 8 * kq);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qf[s] = q_ok ? *(const bf16x8 *)(qrow + (FP8 ? 8 * s : 32 * s))
                         : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }

    // Byte addressing. Consecutive keys of one K/V head are row_bytes apart
    // (contiguous cache: [B, Sk, Hkv, D]; paged: [pages, block, Hkv, D]).
    // Lane bases fold in the head and the lane's fixed column.
    const int64_t row_bytes = (int64_t)p.Hkv * D * ESZ;
    const int64_t head_off = (int64_t)kvh * D * ESZ + (PAGED ? 0 : (int64_t)b * p.Sk * row_bytes);
    const unsigned char *kbase =
        (const unsigned char *)p.k + head_off + (FP8 ? 8 * NS * kq : 8 * kq) * ESZ;
    const unsigned char *vbase = (const unsigned char *)p.v + head_off + (lane % VCPR) * 16;
    const int lb = PAGED ? p.log2_block : 0;
    const int64_t page_bytes = row_bytes << lb;
    const int slot_mask = (1 << lb) - 1;
    int tbl_lo = 0;
    // Address of key `key` (which must lie in the staged table window when paged).
    auto key_ptr = [&](const unsigned char *base, int key) -> const unsigned char * {
        if constexpr (PAGED) {
            const int page = tbl[(key >> lb) - tbl_lo];
            return base + page * page_bytes + (int64_t)(key & slot_mask) * row_bytes;
        } else {
            return base + (int64_t)key * row_bytes;
        }
    };
    __bf16 *vsw = (__bf16 *)smem + wave * TK * VRS;  // this wave's V tile, row-major bf16

    kraw_t kf[2][NS], kf_n[2][NS];
    u32x4 vreg[NVL], vreg_n[NVL];
    int w_hi = k_hi;  // end of the current table window

    // Tile t0's K rows (keys t0 + 16 kt + qi) and V rows (16-byte chunk lane + 64 i
    // of the tile), clamped into [k_lo, w_hi); clamped rows are masked below.
    auto load = [&](int t0, kraw_t (&kd)[2][NS], u32x4 (&vd)[NVL]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const unsigned char *krow = key_ptr(kbase, min(t0 + 16 * kt + qi, w_hi - 1));
            if constexpr (FP8) {
                // the lane's 8 NS codes are contiguous: 16-byte loads
#pragma unroll
                for (int h = 0; h < NS / 2; ++h) {
                    const u32x4 w = load_kv<u32x4, false>(krow + 16 * h);
                    kd[kt][2 * h] = kraw_t{w[0], w[1]};
                    kd[kt][2 * h + 1] = kraw_t{w[2], w[3]};
                }
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s) kd[kt][s] = load_kv<kraw_t, false>(krow + 32 * s * ESZ);
            }
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int key = min(t0 + lane / VCPR + i * (64 / VCPR), w_hi - 1);
            vd[i] = load_kv<u32x4, true>(key_ptr(vbase, key));
        }
    };
    auto k_operand = [&](const kraw_t &raw) -> bf16x8 {
        if constexpr (FP8) {
            const u32x2 lo = fp8x4_to_bf16x4(raw[0]), hi = fp8x4_to_bf16x4(raw[1]);
            return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        } else {
            return raw;
        }
    };
    // PV operand: in 16-lane group kq, lane j reads row 4 kq + j/4 (+16 for
    // the second read), columns 16 dt + 4 (j%4) .. +3; ds_read_b64_tr_b16
    // then gives lane j the column 16 dt + j of those 4 rows.
    const int v_rd = (4 * kq + (qi >> 2)) * VRS + 4 * (qi & 3);

    const float c = p.scale_log2;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{};

    // Paged caches stage the block-table entries of a window of at most
    // MAX_TBL blocks in LDS and walk the split window by window (one window
    // unless the split spans more than MAX_TBL blocks); contiguous caches
    // have a single window.
    for (int w_lo = k_lo; w_lo < k_hi; w_lo = w_hi) {
        if constexpr (PAGED) {
            tbl_lo = w_lo >> lb;
            w_hi = (int)min((int64_t)k_hi, ((int64_t)tbl_lo + MAX_TBL) << lb);
            const int nblk = ((w_hi - 1) >> lb) - tbl_lo + 1;
            __syncthreads();  // every wave is done with the previous window's entries
            for (int i = tid; i < nblk; i += NTHREADS)
                tbl[i] = p.block_table[(int64_t)b * p.max_blocks + tbl_lo + i];
            __syncthreads();
        }
        int t0 = w_lo + TK * wave;
        if (t0 < w_hi) load(t0, kf, vreg);
        for (; t0 < w_hi; t0 += TK * NWAVES) {
            // V tile -> this wave's LDS slice, row-major bf16.
#pragma unroll
            for (int i = 0; i < NVL; ++i) {
                const int c8 = lane + 64 * i;
                __bf16 *dst = vsw + (c8 / VCPR) * VRS + (c8 % VCPR) * VCH;
                if constexpr (FP8) {
                    const u32x2 a = fp8x4_to_bf16x4(vreg[i][0]), b2 = fp8x4_to_bf16x4(vreg[i][1]);
                    const u32x2 c2 = fp8x4_to_bf16x4(vreg[i][2]), d2 = fp8x4_to_bf16x4(vreg[i][3]);
                    *(u32x4 *)dst = u32x4{a[0], a[1], b2[0], b2[1]};
                    *(u32x4 *)(dst + 8) = u32x4{c2[0], c2[1], d2[0], d2[1]};
                } else {
                    *(u32x4 *)dst = vreg[i];
                }
            }
            const int tn = t0 + TK * NWAVES;
            if (tn < w_hi) load(tn, kf_n, vreg_n);

            // S^T = K Q^T: 2 tiles of 16 keys x 16 query heads.
            f32x4 sacc[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sacc[kt] = f32x4{};
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(kf[kt][s]), qf[s],
                                                                       sacc[kt], 0, 0, 0);
            }
            if (t0 + TK > w_hi) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (t0 + 16 * kt + 4 * kq + r >= w_hi) sacc[kt][r] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = pair_max32(mx);
            // Move the reference max only when it is exceeded by more than
            // kRescaleGap (see fwd_bf16.hip); the result is unchanged.
            const float mxs = mx * c;
            if (mxs > m_run + kRescaleGap) {
                const float alpha = fast_exp2(m_run - mxs);
                m_run = mxs;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < NDT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[i][r] *= alpha;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
            bf16x8 pf;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pv = fast_exp2(fmaf(sacc[kt][r], c, -m_use));
                    l_run += pv;
                    pf[4 * kt + r] = (__bf16)pv;
                }

            // O^T += V^T P^T; k-slot j of lane (qi, kq) is key 16*(j/4) + 4*kq + j%4.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int i = 0; i < NDT; ++i) {
                const __bf16 *vp = vsw + 16 * i + v_rd;
                const u32x2 lo = lds_read_tr16(vp);
                const u32x2 hi = lds_read_tr16(vp + 16 * VRS);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                oacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[i], 0, 0, 0);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            if (tn < w_hi) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int s = 0; s < NS; ++s) kf[kt][s] = kf_n[kt][s];
#pragma unroll
                for (int i = 0; i < NVL; ++i) vreg[i] = vreg_n[i];
            }
        }
    }

    // Sum this wave's l over the 4 lanes that share a query.
    l_run += __shfl_xor(l_run, 16);
    l_run = pair_sum32(l_run);

    // Merge the 4 waves' (m, l, O^T) through LDS.
    __syncthreads();
    float *mo = (float *)smem;               // [wave][d][16]
    float *mm = mo + NWAVES * D * 16;        // [wave][16]
    float *ml = mm + NWAVES * 16;            // [wave][16]
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) mo[(wave * D + 16 * i + 4 * kq + r) * 16 + qi] = oacc[i][r];
    if (kq == 0) {
        mm[wave * 16 + qi] = m_run;
        ml[wave * 16 + qi] = l_run;
    }
    __syncthreads();

    for (int idx = tid; idx < 16 * D; idx += NTHREADS) {
        const int q2 = idx / D, d = idx - q2 * D;
        const int g2 = qs * 16 + q2;
        if (g2 >= p.G) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) M = fmaxf(M, mm[w * 16 + q2]);
        float o = 0.f, l = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) {
                const float f = fast_exp2(mm[w * 16 + q2] - M);
                l += f * ml[w * 16 + q2];
                o += f * mo[(w * D + d) * 16 + q2];
            }
        }
        const bool empty = !(l > 0.f);
        const float val = empty ? 0.f : o / l * p.v_scale;
        const float lse = empty ? -INFINITY : (M + log2f(l)) * kLn2;
        const int64_t row = (int64_t)b * p.Hq + kvh * p.G + g2;
        if (p.num_splits == 1) {
            ((__bf16 *)p.o)[row * D + d] = (__bf16)val;
            if (d == 0) p.lse[row] = lse;
        } else {
            const int64_t prow = (int64_t)split * rows + row;
            p.ws_o[prow * D + d] = val;
            if (d == 0) p.ws_lse[prow] = lse;
        }
    }
}

// Merge num_splits partials per (batch, head) row: one wavefront per row.
// Lane s reads L_s (num_splits <= 64), so the max M and the weights
// w_s = exp(L_s - M) (0 for an empty split) come from one load per lane and
// fixed-order shuffle trees; then the lanes sum w_s O_s over s in split
// order with the row's O_s loads unrolled and independent, so the merge pays
// about one memory latency rather than one per split. An empty split's O_s
// is never written: it is read (inside the workspace) but multiplied by
// nothing (selected to 0).
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ ws_o,
                                                      const float *__restrict__ ws_lse,
                                                      void *out, float *lse, int rows, int ns) {
    constexpr int PER = D / 64;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float *src = ws_o + (int64_t)row * D + lane;
    const int64_t split_stride = (int64_t)rows * D;
    // the O_s of the first PRE splits are loaded together with the L_s (split
    // index clamped into the workspace; splits past ns get weight 0), so that
    // both arrive after one memory latency
    constexpr int PRE = 8;
    float pre[PRE][PER];
#pragma unroll
    for (int s = 0; s < PRE; ++s)
#pragma unroll
        for (int e = 0; e < PER; ++e) pre[s][e] = src[min(s, ns - 1) * split_stride + 64 * e];
    const float ls = lane < ns ? ws_lse[(int64_t)lane * rows + row] : -INFINITY;
    float M = ls;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = (ls == -INFINITY) ? 0.f : __expf(ls - M);
    float tot = w;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < PRE; ++s) {
        const float ws = __shfl(w, s);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(ws, ws != 0.f ? pre[s][e] : 0.f, acc[e]);
    }
#pragma unroll 8
    for (int s = PRE; s < ns; ++s) {
        const float ws = __shfl(w, s);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const float v = src[s * split_stride + 64 * e];
            acc[e] = fmaf(ws, ws != 0.f ? v : 0.f, acc[e]);
        }
    }
    const bool empty = !(tot > 0.f);
    const float inv = empty ? 0.f : 1.f / tot;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const float val = acc[e] * inv;
        if (OUT_BF16)
            ((__bf16 *)out)[(int64_t)row * D + lane + 64 * e] = (__bf16)val;
        else
            ((float *)out)[(int64_t)row * D + lane + 64 * e] = val;
    }
    if (lane == 0) lse[row] = empty ? -INFINITY : M + logf(tot);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams &p, int d, bool paged, bool fp8_kv, hipStream_t s) {
    const long long grid = (long long)p.B * p.Hkv * p.num_splits * p.n_qs;
#define GQA_CASE(D_, P_, F_)                                                                      \
    if (d == D_ && paged == P_ && fp8_kv == F_) {                                                 \
        hipLaunchKernelGGL((decode_bf16_kernel<D_, P_, F_>), dim3((unsigned)grid), dim3(NTHREADS), \
                           0, s, p);                                                              \
        return hipGetLastError();                                                                 \
    }
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

hipError_t launch_decode_combine(const float *ws_o, const float *ws_lse, void *out, float *lse,
                                 int rows, int num_splits, int d, bool out_bf16, hipStream_t s) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
#define GQA_CASE(D_, B_)                                                                        \
    if (d == D_ && out_bf16 == B_) {                                                            \
        hipLaunchKernelGGL((combine_kernel<D_, B_>), dim3(grid), dim3(256), 0, s, ws_o, ws_lse, \
                           out, lse, rows, num_splits);                                         \
        return hipGetLastError();                                                               \
    }
    GQA_CASE(64, true)
    GQA_CASE(64, false)
    GQA_CASE(128, true)
    GQA_CASE(128, false)
#undef GQA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gqa
