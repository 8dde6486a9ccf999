// Fused GQA attention forward, bf16 in / bf16 out, on gfx950 matrix cores;
// the same kernel with its F8 flag set serves fp8 e4m3 inputs (see the note
// above the kernel template).
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
// works"): a workgroup's row tile holds all G query heads of one K/V head,
// row rho = position * G + head_in_group, so every K/V tile brought on chip is
// used by the whole group. The query-head -> K/V-head map is fixed per
// workgroup before the loop.
//
// gfx950 mapping (our design, not the pages'):
//  * 4 (d = 64) or 8 (d = 128) wavefronts x 32 packed rows;
//    v_mfma_f32_32x32x16_bf16 computes the
//    transposed score tile S^T = K Q^T so that each lane owns one query row:
//    a row max or row sum is in-lane plus one v_permlane32_swap.
//  * O^T = V^T P^T accumulates with the same lane <-> query ownership, so the
//    rescale by exp(m_old - m_new) is a per-lane scalar multiply and P never
//    leaves registers (its bf16 copy is the B operand as produced).
//  * The reference max m is the exact max of tile 0 and moves only when a
//    tile's probabilities grow past a bound (then that tile is recomputed
//    against the raised m); any reference gives the same result, since m
//    cancels between O~ and l and is added back in L.
//  * K and V are staged row-major in LDS by direct global->LDS loads of whole
//    rows (no staging registers) into a 4-slot ring per tensor, 3 tiles
//    ahead; the V^T operand is read with ds_read_b64_tr_b16, which hands each
//    lane a column slice. Software-pipelined: the scores of tile t+1 run on
//    the matrix cores while the vector units exponentiate tile t (one barrier
//    per tile, one code path: every wave runs every tile of its workgroup,
//    masked where it lies past the wave's causal limit).
//  * exp is 2^x on the transcendental unit with scale*log2(e) folded into one
//    FMA; P and O are rounded to bf16 with round-to-nearest-even.
//  * Workgroup order: the row tiles of a head group run back to back on one
//    XCD (workgroups are dealt round-robin to the 8 XCDs), so its K/V comes
//    from HBM once and is then reused from that XCD's L2; causal row tiles are
//    issued heaviest first.

#include <type_traits>

#include "device_util.h"
#include "params.h"

namespace gqa {

namespace {

#ifndef GQA_BN128
#define GQA_BN128 32
#endif
#ifndef GQA_PF_K
#define GQA_PF_K 6
#endif
#ifndef GQA_VR_DIV
#define GQA_VR_DIV 1
#endif

// Wavefronts per workgroup (32 query rows each): 8 at d = 128, where sharing
// each K/V tile among 256 rows measured 3-5 % faster than 128 rows, 4 at
// d = 64, where 8 waves measured 15 % slower on the encoder workload.
template <int D>
struct Waves {
    static constexpr int NW = D == 128 ? 8 : 4;
    static constexpr int BM = 32 * NW;        // packed query rows per workgroup
    static constexpr int NTHREADS = 64 * NW;
};

// K and V tiles live in LDS as unpadded row-major [key][d] bf16, filled by
// direct global->LDS loads (global_load_lds_dwordx4: one wavefront
// instruction writes 64 x 16 contiguous bytes). Bank conflicts are avoided by
// an XOR swizzle of the 16-byte chunk index within each row: chunk c of row r
// sits in slot c ^ swz(r). The K swizzle spreads the 32 rows read by one
// matrix-core operand load over all banks; the V swizzle does the same for
// the 4-row x 32-byte footprint of each transposing read.
template <int D>
struct Cfg {
    static constexpr int NW = Waves<D>::NW;
    // 32 keys per tile. At d = 128 this keeps two score tiles, the output
    // accumulator and the Q fragment within 256 VGPRs (2 waves/SIMD); at
    // d = 64 within 168 VGPRs and 48 KiB of LDS, so three workgroups share a
    // CU (3 waves/SIMD), which measured 6-7 % faster on the encoder shape
    // than 64-key tiles at 2 waves/SIMD.
    static constexpr int BN = D == 128 ? GQA_BN128 : 32;
    static constexpr int C8 = D / 8;                    // 16-byte chunks per row
    static constexpr int NDMA = BN * D * 2 / 1024 / NW;  // DMA instructions per wave per tensor
    static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    // fp8 rows (D bytes, C16 = D / 16 chunks): 16 consecutive rows read at
    // one chunk hit distinct bank groups (two rows per 256 bytes at d = 128,
    // four at d = 64).
    static __device__ __forceinline__ int swz8(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
    static __device__ __forceinline__ int swz_v(int r) {
        return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
    }
};

// F8: q, k, v hold fp8 e4m3 codes (one byte each) with per-tensor
// dequantisation scales folded into scale_log2 (q_scale k_scale) and o_scale
// (v_scale). The scores run on the fp8 matrix cores (32x32x64: exact
// products; each group of 64 is summed inside the matrix core at somewhat
// less than fp32 precision, then accumulated in fp32). K and V tiles arrive together, one 16-byte direct load per
// wave (half of the waves fetch K rows, half V rows), into one ring slot: K in
// its lower half (fp8 rows, swizzled for the operand reads), V in its upper
// half (unswizzled). One step before its use, the workgroup widens the V tile
// exactly to bf16 into one of two bf16 V slots, so P stays bf16 and O^T += V^T
// P^T runs as in the bf16 kernel: the result is the attention of the
// dequantised inputs, rounded as in the bf16 path.
template <int D, bool CAUSAL, bool VARLEN, bool F8>
__global__ __launch_bounds__(Waves<D>::NTHREADS) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2))) void
fwd_bf16_kernel(FwdParams p) {
    using CF = Cfg<D>;
    constexpr int NW = Waves<D>::NW, BM = Waves<D>::BM;
    constexpr int BN = CF::BN, C8 = CF::C8, NDMA = CF::NDMA;
    constexpr int DSTEPS = D / 16;  // k-steps of the score product
    constexpr int DBLK = D / 32;    // 32-row blocks of O^T
    constexpr int KB = BN / 32;     // 32-key blocks per tile

    // A 4-slot LDS ring per tensor (tile j in slot j % 4), one array per slot
    // so that DMA in flight into one slot is visibly disjoint from reads of
    // another; slot indices are compile-time constants in every step.
    __shared__ __attribute__((aligned(1024))) __bf16 Ks0[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 Ks1[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 Ks2[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 Ks3[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 Vs0[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 Vs1[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 Vs2[F8 ? 8 : BN * D];  // F8: two bf16 V slots
    __shared__ __attribute__((aligned(1024))) __bf16 Vs3[F8 ? 8 : BN * D];
    // The workgroup's Q rows, staged once by the same direct loads (K swizzle).
    __shared__ __attribute__((aligned(1024))) __bf16 Qs[BM * D];
    auto kslot = [&](auto j) -> __bf16 * {
        constexpr int J = decltype(j)::value & 3;
        return J == 0 ? Ks0 : J == 1 ? Ks1 : J == 2 ? Ks2 : Ks3;
    };
    auto vslot = [&](auto j) -> __bf16 * {
        constexpr int J = decltype(j)::value & (F8 ? 1 : 3);
        return J == 0 ? Vs0 : J == 1 ? Vs1 : J == 2 ? Vs2 : Vs3;
    };

    const int tid = threadIdx.x;
    // the wave index is wave-uniform: kept in a scalar register so that the
    // per-wave conditions below are scalar branches, not lane masks
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
        if constexpr (F8 && D == 64) {
            // A 64-byte fp8 row fills half of a 128-byte line whose other
            // half is the same token's row of the next head group: XCD x
            // runs head groups 16 a + 2 x and 16 a + 2 x + 1 at the same
            // time, so both halves of each line are used from its L2.
            if ((p.n_hg & 15) == 0) hg = (hg >> 4) * 16 + (hg & 7) * 2 + ((hg >> 3) & 1);
        }
    } else {
        hg = pid / p.n_rb;
        rank = pid % p.n_rb;
    }
    const int rb = CAUSAL ? (p.n_rb - 1 - rank) : rank;
    const int hpb = p.Hq / p.gpack;
    const int seq_rank = hg / hpb;
    const int qh0 = (hg - seq_rank * hpb) * p.gpack;
    int b = seq_rank;
    // Longest first (packed batches of 2 .. kLptMax sequences): the heaviest
    // row tiles start first and short sequences fill the tail.
    if constexpr (VARLEN) {
        if (p.B > 1 && p.B <= kLptMax) b = lpt_sequence(p.cu_q, p.cu_k, p.B, seq_rank, tid);
    }
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

    // ---- this wave's rows: from which key on its tiles need masking ----
    // Every wave runs every tile of the workgroup (one path, no per-wave
    // branches in the loop). A tile that lies wholly past a wave's causal
    // limit is masked to -inf, so it adds nothing: p = 0 and no max moves.
    // Rows past the end hold clamped copies of the last row and are never
    // stored.
    const int wave_kfull = CAUSAL ? min(Lk, (row0 + wave * 32) / p.gpack + 1 + shift) : Lk;

    // ---- Q fragment (B operand of S^T = K Q^T), kept in registers ----
    // It arrives through LDS: its direct loads are issued just before the
    // first K/V tiles and waited for together with them, so the workgroup's
    // start pays one memory latency rather than the Q load's and then the
    // first tiles'. Rows past the end are clamped to the last row (finite
    // values whose results are never stored).
    bf16x8 qf[F8 ? 1 : DSTEPS];
    constexpr int DS8 = D / 64;  // F8: k-steps of the fp8 score product
    i32x8 qf8[F8 ? DS8 : 1];

    const int64_t kv_stride = (int64_t)p.Hkv * D;
    const __bf16 *kbase = (const __bf16 *)p.k + ((int64_t)k_tok0 * p.Hkv + kvh) * D;
    const __bf16 *vbase = (const __bf16 *)p.v + ((int64_t)k_tok0 * p.Hkv + kvh) * D;

    // DMA staging: instruction i of wave w fills LDS bytes [1024 (w + NW i), +1024)
    // of a tile; lane l of it covers chunk slot (64 (w + NW i) + l) % C8 of row
    // (64 (w + NW i) + l) / C8 and fetches the global chunk that belongs there.
    // A tile is addressed as a wave-uniform base (scalar arithmetic) plus a
    // 32-bit per-lane byte offset. Rows past kend are clamped to the last
    // needed key, and steps past the last needed tile (issued so that every
    // step has the same number of loads) re-load it: real, finite K/V rows
    // whose scores are masked to -inf or never used.
    const uint32_t row_bytes = (uint32_t)kv_stride * 2;  // < 2^24 (Hkv d <= 2^22)
    const uint32_t tile_bytes = BN * row_bytes;
    auto dma_kv = [&](const __bf16 *base, int t, auto is_v, __bf16 *dst) {
        const int tt = min(t, ntiles - 1);   // a tile holding needed keys
        const int last = kend - 1 - tt * BN;  // its last needed row (>= 0)
        const char *tile = (const char *)base + (uint64_t)(uint32_t)tt * tile_bytes;
        const uint32_t lds0 = lds_addr(dst) + 1024 * wave;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int idx = 64 * (wave + NW * i) + lane;
            const int r = idx / C8;
            const int sw = decltype(is_v)::value ? CF::swz_v(r) : CF::swz_k(r);
            const uint32_t ch_bytes = ((idx % C8) ^ sw) * 16;
            lds_dma16_sv(tile, __umul24((uint32_t)min(r, last), row_bytes) + ch_bytes,
                         lds0 + 1024 * NW * i);
        }
    };
    auto dma_k = [&](int t, __bf16 *dst) { dma_kv(kbase, t, std::false_type{}, dst); };
    auto dma_v = [&](int t, __bf16 *dst) { dma_kv(vbase, t, std::true_type{}, dst); };
    // Barrier that lets the two most recent DMA groups (2 x 2 NDMA loads per
    // wave) stay in flight: everything older has landed in LDS for this wave,
    // and after s_barrier for every wave. No release fence (which would drain
    // all outstanding loads); the asm is a compiler memory barrier.
    static_assert(NDMA == 1 || NDMA == 2, "barrier wait count assumes 1 or 2 DMA loads per tensor");
    auto barrier_keep2 = [] {
        if constexpr (NDMA == 2)
            asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    auto barrier_lds = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    // d = 64: near the end of the loop no DMA is issued for tiles past the
    // last needed one (the prologue still loads tiles 0-3 and 0-2, clamped):
    // the barrier then keeps in flight only the loads actually issued after
    // K(t+2) and V(t+1), and the workgroup ends with nothing left to drain
    // (1-2 % faster at d = 64; at d = 128 the extra branches cost more than
    // they save).
    constexpr bool TAIL_SKIP = D == 64 && !F8;
    static_assert(NDMA == 1, "the tail wait counts assume one DMA load per tensor and step");
    // F8: K and V tile t into ring slot dst (K rows in its first BN D bytes,
    // V rows in the next BN D bytes): wave w < NW/2 fetches 1024 bytes of K,
    // wave NW/2 + w the same bytes of V; lane l covers 16-byte chunk
    // (64 w' + l) % C16 of row (64 w' + l) / C16. K chunks are swizzled (slot
    // c ^ swz8(r)), V chunks are not. Rows past kend are clamped as above.
    constexpr int C16 = D / 16;  // 16-byte chunks per fp8 row
    static_assert(!F8 || BN * D == 1024 * (NW / 2), "F8: one 16-byte load per wave and tile");
    const uint32_t row_bytes8 = (uint32_t)kv_stride;  // fp8 row stride
    const bool kv_is_v = wave >= NW / 2;               // wave-uniform
    const int wk = kv_is_v ? wave - NW / 2 : wave;
    const unsigned char *kv8base =
        (const unsigned char *)(kv_is_v ? p.v : p.k) + ((int64_t)k_tok0 * p.Hkv + kvh) * D;
    const int dma8_r = (64 * wk + lane) / C16;
    const uint32_t dma8_c = (uint32_t)((((64 * wk + lane) % C16) ^ (kv_is_v ? 0 : CF::swz8(dma8_r))) * 16);
    auto dma_kv8 = [&](int t, __bf16 *dst) {
        const int tt = min(t, ntiles - 1);
        const int last = kend - 1 - tt * BN;
        const unsigned char *tile = kv8base + (uint64_t)(uint32_t)tt * (BN * row_bytes8);
        const uint32_t lds0 = lds_addr(dst) + (kv_is_v ? BN * D : 0) + 1024 * wk;
        lds_dma16_sv(tile, __umul24((uint32_t)min(dma8_r, last), row_bytes8) + dma8_c, lds0);
    };
    // F8: the two most recent KV groups (one load each) may stay in flight.
    auto barrier_keep2_f8 = [] { asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    // F8: widen V tile j (upper half of its ring slot, fp8) to bf16 in its V
    // slot: thread x converts 8 values, row x / (D/8), elements 8 (x % (D/8)) ..
    const int cv_row = tid / (D / 8), cv_part = tid % (D / 8);
    static_assert(!F8 || Waves<D>::NTHREADS * 8 == BN * D, "F8: 8 V values per thread and tile");
    auto widen_v = [&](const __bf16 *slot, __bf16 *vdst) {
        const u32x2 raw = *(const u32x2 *)((const unsigned char *)slot + BN * D + tid * 8);
        const u32x2 lo = fp8x4_to_bf16x4(raw[0]), hi = fp8x4_to_bf16x4(raw[1]);
        *(u32x4 *)(vdst + cv_row * D + ((cv_part ^ CF::swz_v(cv_row)) * 8)) = u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    auto barrier_tail = [](int keep) {
        if (keep >= 4)
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else if (keep == 3)
            asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else if (keep == 2)
            asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else if (keep == 1)
            asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // K operand (A of S^T = K Q^T): row kb*32 + col, chunk 2 s + half.
    int k_rd[DSTEPS];
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) k_rd[s] = col * D + (((2 * s + half) ^ CF::swz_k(col)) * 8);
    // F8 operand of k-step s: row col, bytes 64 s + 32 half .. +31 (logical
    // chunks 4 s + 2 half and + 1), the same for K and Q so that the lanes'
    // k indices of both operands agree; byte offsets.
    int k8_rd[F8 ? 2 * DS8 : 1];
    if constexpr (F8) {
#pragma unroll
        for (int s = 0; s < DS8; ++s)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                k8_rd[2 * s + e] = col * D + (((4 * s + 2 * half + e) ^ CF::swz8(col)) * 16);
    }
    // V^T operand through ds_read_b64_tr_b16: in 16-lane group g, lane j reads
    // row key0 + j/4, columns d0 + 4 (j%4) .. +3 and receives column d0 + j of
    // rows key0 .. key0+3, with d0 = 32 i + 16 (g & 1) and key0 = 4 (g >> 1)
    // (+ 8 for the second read) inside the 16-key slot.
    const int vj = lane & 15, vg = lane >> 4;
    const int v_row = 4 * (vg >> 1) + (vj >> 2);
    int v_rd[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) {
        const int chunk = 4 * i + 2 * (vg & 1) + ((vj & 3) >> 1);
        v_rd[i] = v_row * D + ((chunk ^ CF::swz_v(v_row)) * 8) + 4 * (vj & 1);
    }

    const float c = p.scale_log2;
    float m_run = -INFINITY;  // reference max of scaled scores, log2 units
    float l_run = 0.f;        // this lane's share of the running sum
    f32x16 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};

    // S^T tile (rows = keys, columns = this wave's 32 query rows) from LDS.
    auto scores = [&](const __bf16 *ks, f32x16 (&sacc)[KB]) {
        if constexpr (F8) {
            const unsigned char *k8 = (const unsigned char *)ks;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                sacc[kb] = f32x16{};
#pragma unroll
                for (int s = 0; s < DS8; ++s) {
                    const u32x4 lo = *(const u32x4 *)(k8 + kb * 32 * D + k8_rd[2 * s]);
                    const u32x4 hi = *(const u32x4 *)(k8 + kb * 32 * D + k8_rd[2 * s + 1]);
                    const i32x8 a = __builtin_bit_cast(
                        i32x8, u32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                    // formats 0 / 0: both operands fp8 e4m3; E8M0 scales 127 = 1
                    sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[s], sacc[kb], 0, 0,
                                                                              0, 127, 0, 127);
                }
            }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s) {
                const bf16x8 a = *(const bf16x8 *)(ks + kb * 32 * D + k_rd[s]);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
            }
        }
    };
    // Element mask, only on tiles crossing the diagonal or the end, and on the
    // tile past the end whose scores the last step computes.
    auto mask = [&](int t, f32x16 (&sacc)[KB]) {
        if ((t + 1) * BN > wave_kfull || t >= ntiles) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t * BN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (key >= row_kend) sacc[kb][r] = -INFINITY;
                }
        }
    };
    // Move the reference max m up to the tile's row max (when that is larger)
    // and rescale O~ and l by 2^(m_old - m_new).
    auto raise_max = [&](const f32x16 (&sacc)[KB]) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        const float mxs = pair_max32(mx) * c;
        if (mxs > m_run) {
            const float alpha = fast_exp2(m_run - mxs);
            m_run = mxs;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DBLK; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        }
    };
    // p = 2^(s c - m) in fp32, summed into l_tile and rounded to bf16 as the B
    // operand.
    auto probs = [&](const f32x16 (&sacc)[KB], bf16x8 (&pf)[KB][2], float &l_tile) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        l_tile = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pv = fast_exp2(fmaf(sacc[kb][8 * h2 + j], c, -m_use));
                    l_tile += pv;
                    pf[kb][h2][j] = (__bf16)pv;
                }
    };
    // O^T += V^T P^T. P^T key order in lane (col, half) for k-slot j:
    // key = kb*32 + 16*h2 + 8*(j/4) + 4*half + j%4, matched by the V^T reads.
    auto load_v = [&](const __bf16 *vs, bf16x8 (&vf)[KB][2][DBLK]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < DBLK; ++i) {
                    const __bf16 *vp = vs + (kb * 32 + 16 * h2) * D + v_rd[i];
                    const u32x2 lo = lds_read_tr16(vp);
                    const u32x2 hi = lds_read_tr16(vp + 8 * D);
                    vf[kb][h2][i] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                }
    };
    auto accumulate = [&](const bf16x8 (&vf)[KB][2][DBLK], const bf16x8 (&pf)[KB][2]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < DBLK; ++i)
                    oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb][h2][i], pf[kb][h2],
                                                                     oacc[i], 0, 0, 0);
    };

    // Software pipeline, one barrier per tile, DMA three tiles ahead.
    // Entering step t: K(t+1) and V(t) have landed in LDS, the DMA of K(t+2),
    // K(t+3), V(t+1), V(t+2) may be in flight, and the scores of tile t are
    // masked. Step t starts the DMA of K(t+4) (into K(t)'s slot) and V(t+3)
    // (into V(t-1)'s slot), computes the scores of tile t+1 on the matrix
    // cores while the vector units turn tile t into probabilities (checked
    // against the reference max), accumulates P(t) V(t), masks tile t+1, then
    // waits until K(t+2) and V(t+1) have landed and meets the other waves. Steps past the last
    // needed tile re-load that tile (never used) so that every step issues the
    // same number of DMA loads and the wait count stays exact; the last step
    // also scores K(ntiles), such a re-load, and masks all of it.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    f32x16 sa[KB], sb[KB];
    if (ntiles > 0 && F8) {
        // fp8 Q rows (D bytes each, swizzled as the K rows), then KV(0..3)
        constexpr int NQ8 = BM * D / 1024 / NW;  // Q loads per wave
#pragma unroll
        for (int i = 0; i < NQ8; ++i) {
            const int idx = 64 * (wave + NW * i) + lane;
            const int r = idx / C16;
            const int rho = min(row0 + r, rows_total - 1);
            const int qp = rho / p.gpack;
            const int qh = qh0 + (rho - qp * p.gpack);
            const unsigned char *src = (const unsigned char *)p.q + ((int64_t)(q_tok0 + qp) * p.Hq + qh) * D +
                                       ((idx % C16) ^ CF::swz8(r)) * 16;
            lds_dma16(src, lds_addr(Qs) + 1024 * (wave + NW * i));
        }
        dma_kv8(0, kslot(I0{}));
        dma_kv8(1, kslot(I1{}));
        dma_kv8(2, kslot(I2{}));
        dma_kv8(3, kslot(I3{}));
        barrier_keep2_f8();  // Q, KV(0), KV(1) have landed
        widen_v(kslot(I0{}), vslot(I0{}));
        const unsigned char *q8 = (const unsigned char *)Qs + wave * 32 * D;
#pragma unroll
        for (int s = 0; s < DS8; ++s) {
            const u32x4 lo = *(const u32x4 *)(q8 + k8_rd[2 * s]);
            const u32x4 hi = *(const u32x4 *)(q8 + k8_rd[2 * s + 1]);
            qf8[s] = __builtin_bit_cast(i32x8, u32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
        scores(kslot(I0{}), sa);
        mask(0, sa);
        raise_max(sa);
        barrier_lds();  // V(0) widened; K(0)'s slot is refilled with KV(4) in step 0
    } else if (ntiles > 0) {
        constexpr int NQ = BM * D * 2 / 1024 / NW;  // Q loads per wave
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int idx = 64 * (wave + NW * i) + lane;
            const int r = idx / C8;
            const int rho = min(row0 + r, rows_total - 1);
            const int qp = rho / p.gpack;
            const int qh = qh0 + (rho - qp * p.gpack);
            const __bf16 *src = (const __bf16 *)p.q + ((int64_t)(q_tok0 + qp) * p.Hq + qh) * D +
                                ((idx % C8) ^ CF::swz_k(r)) * 8;
            lds_dma16(src, lds_addr(Qs) + 1024 * (wave + NW * i));
        }
        dma_k(0, kslot(I0{}));
        dma_k(1, kslot(I1{}));
        dma_v(0, vslot(I0{}));
        dma_k(2, kslot(I2{}));
        dma_v(1, vslot(I1{}));
        dma_k(3, kslot(I3{}));
        dma_v(2, vslot(I2{}));
        barrier_keep2();  // Q, K(0), K(1), V(0) have landed
        // this lane's Q row, chunk 2 s + half (same offsets as the K reads)
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) qf[s] = *(const bf16x8 *)(Qs + wave * 32 * D + k_rd[s]);
        scores(kslot(I0{}), sa);
        mask(0, sa);
        raise_max(sa);
        barrier_lds();  // K(0)'s slot is refilled with K(4) in step 0
    }

    auto step = [&](auto jc, int t, f32x16(&s_cur)[KB], f32x16(&s_nxt)[KB]) {
        constexpr int J = decltype(jc)::value;
        __bf16 *k_next = kslot(std::integral_constant<int, J + 1>{});  // K(t+1)
        __bf16 *v_cur = vslot(std::integral_constant<int, J>{});       // V(t)
        const bool tail = TAIL_SKIP && t + 4 >= ntiles;  // within the last four steps
        if constexpr (F8) {
            // KV(t+4) into K(t)'s slot; V(t+1) (landed by the last barrier)
            // widened into the bf16 V slot that V(t-1) used
            dma_kv8(t + 4, kslot(std::integral_constant<int, J>{}));
            widen_v(kslot(std::integral_constant<int, J + 1>{}), vslot(std::integral_constant<int, J + 1>{}));
        } else if (!tail) {
            dma_k(t + 4, kslot(std::integral_constant<int, J>{}));
            dma_v(t + 3, vslot(std::integral_constant<int, J + 3>{}));
        } else if (t + 3 < ntiles) {
            dma_v(t + 3, vslot(std::integral_constant<int, J + 3>{}));
        }
        bf16x8 pf[KB][2];
        bf16x8 vf[KB][2][DBLK];
        float l_tile;
        {
            // The scores of tile t+1 run on the matrix cores while the vector
            // units turn tile t into probabilities: each score MFMA is followed
            // by a slice of the exponentials and of the LDS reads.
            scores(k_next, s_nxt);
            load_v(v_cur, vf);
            probs(s_cur, pf, l_tile);
            constexpr int NSM = KB * (F8 ? DS8 : DSTEPS);  // score MFMAs
            constexpr int NVR = 2 * KB * 2 * DBLK;  // transposing V reads
            constexpr int VALU_PER = (KB * 16 * 7 / 2 + NSM - 1) / NSM;
            __builtin_amdgcn_sched_group_barrier(0x100, GQA_PF_K, 0);
#pragma unroll
            for (int g = 0; g < NSM; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (scores)
                __builtin_amdgcn_sched_group_barrier(0x100, 1 + NVR / NSM / GQA_VR_DIV, 0);  // DS reads
                __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER, 0);  // VALU (exp)
            }
        }
        // The reference m of a row is its exact max over tile 0 (every row that
        // sees any key sees key 0) and then moves only when a tile's
        // probabilities grow large: when some lane's sum over the tile exceeds
        // kTileSumBound (so one p may exceed it), the wave raises m to the tile
        // max, rescales O~ and l, and recomputes the tile. Otherwise every
        // p <= kTileSumBound and no row max is computed. The result is the same
        // for any reference: m cancels between O~ and l and is added back in L.
        if (__builtin_amdgcn_ballot_w64(l_tile > kTileSumBound)) {
            raise_max(s_cur);
            probs(s_cur, pf, l_tile);
        }
        l_run += l_tile;
        accumulate(vf, pf);
        mask(t + 1, s_nxt);
        if constexpr (F8) {
            barrier_keep2_f8();
        } else if (!tail) {
            barrier_keep2();
        } else {
            // loads issued after K(t+2) and V(t+1): K(t+3) and V(t+2) (by the
            // prologue when t = 0), K(t+4) and V(t+3) (only if needed)
            const int keep = (t + 3 < ntiles || t == 0) + (t + 2 < ntiles || t == 0) +
                             (t + 4 < ntiles) + (t + 3 < ntiles);
            barrier_tail(keep);
        }
    };
    int t = 0;
    for (; t + 3 < ntiles; t += 4) {
        step(I0{}, t, sa, sb);
        step(I1{}, t + 1, sb, sa);
        step(I2{}, t + 2, sa, sb);
        step(I3{}, t + 3, sb, sa);
    }
    if (t < ntiles) step(I0{}, t, sa, sb);
    if (t + 1 < ntiles) step(I1{}, t + 1, sb, sa);
    if (t + 2 < ntiles) step(I2{}, t + 2, sa, sb);
    // drain this wave's remaining (unused) DMA before the workgroup can end
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: one division by l, L = m + log(l) ----
    const float l_tot = pair_sum32(l_run);
    const bool empty = !(l_tot > 0.f);
    float inv = empty ? 0.f : 1.f / l_tot;
    if constexpr (F8) inv *= p.o_scale;
    // O leaves through this wave's own 32 rows of Qs (its Q fragment was read
    // from there before the loop; no other wave touches them): lane (col, half)
    // writes its 8-byte pieces of row col, then every lane reads whole 16-byte
    // chunks, so each global store instruction writes 64 x 16 bytes in runs of
    // full D-element rows rather than 32 rows x 16 bytes. Chunk c of row r
    // sits in slot c ^ (r mod C8) to spread the row-strided writes over banks.
    __bf16 *ow = Qs + wave * 32 * D;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[i][4 * g + e] * inv);
            const int c = (4 * i + g) ^ (col & (C8 - 1));
            *(u32x2 *)(ow + col * D + c * 8 + 4 * half) = __builtin_bit_cast(u32x2, w);
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's writes precede its reads
#pragma unroll
    for (int j = 0; j < 32 * C8 / 64; ++j) {
        const int idx = lane + 64 * j;
        const int r = idx / C8, c = idx % C8;
        const u32x4 v = *(const u32x4 *)(ow + r * D + ((c ^ (r & (C8 - 1))) * 8));
        const int rr = row0 + wave * 32 + r;
        if (rr < rows_total) {
            const int rp = rr / p.gpack;
            const int rh = qh0 + (rr - rp * p.gpack);
            *(u32x4 *)((__bf16 *)p.o + ((int64_t)(q_tok0 + rp) * p.Hq + rh) * D + c * 8) = v;
        }
    }
    if (!row_ok) return;
    if (half == 0) {
        const float lse = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
        const int64_t li = VARLEN ? (int64_t)(q_tok0 + pos) * p.Hq + head
                                  : ((int64_t)b * p.Hq + head) * p.Sq + pos;
        p.lse[li] = lse;
    }
}

template <int D, bool CAUSAL, bool VARLEN, bool F8>
hipError_t launch_t(const FwdParams &p, hipStream_t s) {
    const long long grid = (long long)p.n_hg * p.n_rb;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN, F8>), dim3((unsigned)grid),
                       dim3(Waves<D>::NTHREADS), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

int fwd_bf16_rows_per_tile(int d) { return d == 128 ? Waves<128>::BM : Waves<64>::BM; }

hipError_t launch_fwd_bf16(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s) {
#define GQA_CASE(D_, C_, V_) \
    if (d == D_ && causal == C_ && varlen == V_) return launch_t<D_, C_, V_, false>(p, s);
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

hipError_t launch_fwd_fp8(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s) {
#define GQA_CASE(D_, C_, V_) \
    if (d == D_ && causal == C_ && varlen == V_) return launch_t<D_, C_, V_, true>(p, s);
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
