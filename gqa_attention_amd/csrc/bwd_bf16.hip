// Attention backward, bf16 in / bf16 out, on gfx950 matrix cores.
//
// Method (FlashAttention-2 summary, azimuth.plus, paragraph on the backward
// pass): the probabilities are recomputed from the inputs and the stored row
// statistic L (so no S or P is ever stored), key/value gradients are
// accumulated per block of keys, and for grouped heads the key and value
// gradients are the sums over the query heads that share them. With
// P = exp(scale q k^T - L), D = rowsum(dO * O):
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
// (D = rowsum(P * dP) because O = P V; the page prints no formulas.)
//
// gfx950 mapping (our design, not the pages'):
//  * bwd_dq runs first: a workgroup owns 128 packed rows (like the forward)
//    and walks the key tiles: S^T = K Q^T and dP^T = V dO^T (each lane owns
//    a query row, so L and D are per-lane scalars), dQ^T += K^T dS^T. Before
//    its loop it forms D = rowsum(dO * O) and L in log2 units for its rows
//    and stores them in packed-row order (row rho = pos * G + head in group),
//    so that a tile of 32 packed rows is 128 contiguous bytes for the next
//    pass. The page instead adds dQ atomically from the key-block pass; fp32
//    atomics at this scale (one update per key block per dQ element) would
//    cost more than the second pass's recomputation on this chip.
//  * bwd_dkdv: a workgroup owns 128 keys of one K/V head (32 per wave, held
//    as matrix-core operands in registers) and walks all packed rows of the
//    G query heads of the group, so the GQA sum of dK and dV happens inside
//    the accumulators. Per 32-row tile: S = Q K^T and dP = dO V^T (each lane
//    owns a key), then dV^T += dO^T P and dK^T += Q^T dS, with the
//    transposed operands dO^T and Q^T read by ds_read_b64_tr_b16.
//  * Q/dO and K/V tiles stream through an LDS ring (3 slots; 2 for Q/dO at
//    d = 128) with direct global->LDS loads issued ahead, one barrier per
//    tile. Rows are unpadded with an XOR swizzle of the 16-byte chunk index
//    chosen so that both the row-slice reads and the transposing reads of a
//    tile are free of bank conflicts.
//  * One code path per tile in both kernels: every wave runs every tile of
//    its workgroup, with the element mask (a wave-uniform branch) only where
//    the causal diagonal or a ragged end crosses the tile. Under a causal
//    mask a dK/dV workgroup takes key block i and then n_kb - 1 - i, so the
//    workgroups walk about the same number of rows.

#include "device_util.h"
#include "params.h"

namespace gqa {

namespace {

constexpr int NW = 4;  // wavefronts per workgroup
constexpr int NTHREADS = 64 * NW;
constexpr int NSLOT = 3;  // LDS ring depth (tiles two ahead)


// 16-byte chunk slot of chunk c in row r: c ^ swz(r). d = 128 (16 chunks a
// row): 16 consecutive rows read at one chunk hit 16 distinct slots, and the
// 4-row x 2-chunk footprint of a transposing read also hits distinct slots.
// d = 64 (8 chunks, two rows per 256 bytes): the same for rows of equal parity.
template <int D>
__device__ __forceinline__ int swz(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Wait until at most N of this wave's loads are outstanding, then meet the
// other waves (the asm is a compiler memory barrier; no release fence).
template <int N>
__device__ __forceinline__ void wait_barrier() {
    if constexpr (N == 0)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 1)
        asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 2)
        asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 3)
        asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 4)
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 5)
        asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 6)
        asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 10)
        asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        static_assert(N <= 6 || N == 10, "wait count");
}

// Start of head group hgl of sequence b in a workspace array (rows padded to
// a multiple of 4 so that every group starts 16-byte aligned).
__device__ __forceinline__ int64_t ws_base(const BwdParams &p, int b, int hgl) {
    return ((int64_t)b * (p.Hq / p.G) + hgl) * (((int64_t)p.Sq * p.G + 3) & ~(int64_t)3);
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns 128 keys of one K/V head and walks the packed rows.
// ---------------------------------------------------------------------------
// Sequence b's token ranges and the 32-row tiles [t_lo, t_hi) of packed rows
// that see key block kblk (keys kblk*128 ..). Under a causal mask the first
// such row is the first position pos with pos + (Lk - Lq) >= kblk*128.
struct KeyBlockRows {
    int q_tok0, Lq, k_tok0, Lk, t_lo, t_hi;
};
template <bool CAUSAL, bool VARLEN>
__device__ __forceinline__ KeyBlockRows key_block_rows(const BwdParams &p, int b, int kblk) {
    KeyBlockRows r;
    r.q_tok0 = b * p.Sq;
    r.Lq = p.Sq;
    r.k_tok0 = b * p.Sk;
    r.Lk = p.Sk;
    if (VARLEN) {
        r.q_tok0 = p.cu_q[b];
        r.Lq = p.cu_q[b + 1] - r.q_tok0;
        r.k_tok0 = p.cu_k[b];
        r.Lk = p.cu_k[b + 1] - r.k_tok0;
    }
    const int rows_total = r.Lq * p.G;
    int rho_lo = 0;
    if (CAUSAL) rho_lo = min(rows_total, max(0, kblk * 128 - (r.Lk - r.Lq)) * p.G);
    r.t_lo = rho_lo / 32;
    r.t_hi = (rows_total + 31) / 32;
    return r;
}
// Non-empty row chunks of a key block (at least 1: chunk 0 also covers a key
// block that no row sees, whose gradients are zero). At most n_ch, the count
// the workspace holds; the last chunk runs to the end of the rows.
__device__ __forceinline__ int key_block_chunks(const BwdParams &p, const KeyBlockRows &r) {
    if (p.n_ch <= 1) return 1;
    return min(p.n_ch, max(1, (r.t_hi - r.t_lo + p.ch_tiles - 1) / p.ch_tiles));
}

// ONE: the variant for grids of at most one workgroup per CU (a causal
// prefill of one sequence with few K/V heads: B Hkv n_kb / 2 workgroups). Each
// SIMD then runs a single wave, which must hide its own LDS latency: the
// register budget is 512 (one wave per SIMD), V stays in registers at every
// head dim, the ring has 3 slots, and every LDS operand of a tile is read
// ahead of the products that use it.
template <int D, bool CAUSAL, bool VARLEN, bool ONE>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(ONE ? 1 : 2))) void
bwd_dkdv_kernel(BwdParams p) {
    constexpr int BR = 32;             // packed rows per tile
    constexpr int C8 = D / 8;          // 16-byte chunks per row
    constexpr int DSTEPS = D / 16;     // k-steps of the products over head_dim
    constexpr int DBLK = D / 32;       // 32-row blocks of dK^T / dV^T
    constexpr int TILE = BR * D;       // elements of a Q or dO tile
    constexpr int NDQ = TILE * 2 / 1024 / NW;  // loads per wave per Q (or dO) tile
    static_assert(NDQ >= 1, "tile too small for one load per wave");
    constexpr int MISC = 256;          // bytes: L and D of the tile's rows
    constexpr int SLOT = 2 * TILE * 2 + MISC;  // bytes per ring slot
    constexpr int NLOAD = 2 * NDQ + 1;         // loads per wave per tile
    // d = 128: the V operand lives in LDS (its 32 VGPRs would spill next to
    // the two 64-VGPR accumulators), and a 2-slot ring keeps two workgroups
    // per CU; d = 64: V in registers, 3-slot ring.
    constexpr bool VLDS = D == 128 && !ONE;
    // PIPE (ONE): the scores of row tile t + 1 are formed while tile t's
    // probabilities are, so the single wave's matrix core runs under its own
    // exponentials; the ring then holds tile t - 1's slot for the next DMA,
    // tiles t and t + 1 being read, and tile t + 2 in flight (4 slots).
    constexpr bool PIPE = ONE;
    constexpr int NS = VLDS ? 2 : PIPE ? 4 : NSLOT;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 vlds[VLDS ? NW * 32 * D : 8];

    const int tid = threadIdx.x;
    // wave-uniform wave index (scalar register): per-wave conditions are
    // scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_u = wave;

    // ---- workgroup -> (sequence, K/V head, key block, row chunk) ----
    // Key blocks of one (sequence, K/V head) run back to back on one XCD
    // when the pairs split evenly over the 8 XCDs (they share Q and dO
    // through that XCD's L2); lower key blocks (more visible rows under a
    // causal mask) first, and a key block's row chunks together.
    const int pid = blockIdx.x;
    const int n_grp = p.B * p.Hkv;
    const int n_inner = p.pair ? (p.n_kb + 1) / 2 : p.n_kb * p.n_ch;
    int grp, inner;
    if ((n_grp & 7) == 0) {
        const int slot = pid >> 3;
        grp = (slot / n_inner) * 8 + (pid & 7);
        inner = slot % n_inner;
    } else {
        grp = pid / n_inner;
        inner = pid % n_inner;
    }
    const int kvh = grp % p.Hkv;
    int b = grp / p.Hkv;
    if constexpr (VARLEN) {
        // longest first, as the forward; grp follows the sequence taken (the
        // row-chunk partials and their reduction are indexed by it)
        if (p.B > 1 && p.B <= kLptMax) {
            b = lpt_sequence(p.cu_q, p.cu_k, p.B, b, tid);
            grp = b * p.Hkv + kvh;
        }
    }
    // Paired mode (causal, unchunked): key block i and its mirror
    // n_kb(b) - 1 - i, one after the other, so that every workgroup walks
    // about the same number of rows (the first block sees the most rows,
    // its mirror the fewest).
    int npass = 1, kb_first = inner / p.n_ch, chunk = inner - kb_first * p.n_ch, kb_second = -1;
    if (p.pair) {
        const int Lk_b = VARLEN ? p.cu_k[b + 1] - p.cu_k[b] : p.Sk;
        const int nkb = (Lk_b + 127) / 128;
        if (inner >= (nkb + 1) / 2) return;  // uniform over the workgroup
        kb_first = inner;
        chunk = 0;
        kb_second = nkb - 1 - inner;
        npass = kb_second > kb_first ? 2 : 1;
    }
    for (int pass = 0; pass < npass; ++pass) {
    if (pass > 0) __syncthreads();  // every wave is done with the ring and V rows
    int kblk = pass == 0 ? kb_first : kb_second;
    int lane_r = tid & 63;
    // opaque per pass: nothing derived from the lane or the block is kept
    // live across passes (that would raise the register count of the loop)
    asm volatile("" : "+s"(kblk), "+v"(lane_r));
    const int lane = lane_r, col = lane & 31, half = lane >> 5;
    const KeyBlockRows kr = key_block_rows<CAUSAL, VARLEN>(p, b, kblk);
    const int q_tok0 = kr.q_tok0, Lq = kr.Lq, k_tok0 = kr.k_tok0, Lk = kr.Lk;
    const int k0 = kblk * 128;
    if (k0 >= Lk) continue;  // uniform over the workgroup
    const int n_valid = key_block_chunks(p, kr);
    if (chunk >= n_valid) continue;  // uniform: an empty row chunk
    const int G = p.G;
    const int shift = Lk - Lq;
    const int rows_total = Lq * G;
    // This workgroup's 32-row tiles: the key block's whole range, or one chunk.
    const int t_lo = kr.t_lo + chunk * p.ch_tiles;
    const int t_hi = chunk == n_valid - 1 ? kr.t_hi : t_lo + p.ch_tiles;

    // ---- this lane's key and this wave's key range ----
    const int kk = k0 + 32 * wave + col;
    const bool key_ok = kk < Lk;
    // causal: packed row rho sees key kk iff rho / G + shift >= kk, i.e.
    // rho >= (kk - shift) G
    const int row_min = (kk - shift) * G;
    const int wk0 = k0 + 32 * wave;             // first key of this wave
    const int wk1 = min(wk0 + 31, Lk - 1);      // last valid key of this wave

    // K and V rows of this lane's key as B operands (k = head_dim elements
    // 16 s + 8 half .. +7); keys past the end read the last key and are zeroed.
    bf16x8 kf[DSTEPS], vf[VLDS ? 1 : DSTEPS];
    __bf16 *vw = vlds + (VLDS ? wave * 32 * D : 0);  // this wave's V rows (d = 128)
    {
        const int kr = key_ok ? kk : Lk - 1;
        const int64_t off = ((int64_t)(k_tok0 + kr) * p.Hkv + kvh) * D + 8 * half;
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) {
            const u32x4 a = *(const u32x4 *)((const __bf16 *)p.k + off + 16 * s);
            const u32x4 c2 = *(const u32x4 *)((const __bf16 *)p.v + off + 16 * s);
            kf[s] = __builtin_bit_cast(bf16x8, key_ok ? a : u32x4{0u, 0u, 0u, 0u});
            const u32x4 vv = key_ok ? c2 : u32x4{0u, 0u, 0u, 0u};
            if constexpr (VLDS)  // row col, chunk 2 s + half, swizzled as the tiles
                *(u32x4 *)(vw + col * D + (((2 * s + half) ^ swz<D>(col)) * 8)) = vv;
            else
                vf[s] = __builtin_bit_cast(bf16x8, vv);
            x ^= __builtin_bit_cast(u32x4, kf[s]) ^ vv;
        }
        // Consume the loads before the first DMA (see the forward kernel).
        asm volatile("" ::"v"(x[0] ^ x[1] ^ x[2] ^ x[3]));
    }

    // ---- DMA of tile t (packed rows t*32 ..) into a ring slot ----
    // Q and dO rows: instruction i of wave w fills bytes [1024 (w + NW i), +1024)
    // of the tile; lane l covers chunk slot (64 (w + NW i) + l) % C8 of row
    // (64 (w + NW i) + l) / C8. Rows past the end are clamped to the last row.
    // L and D: lanes 0-1 of every wave fetch L of rows 8 w .. 8 w + 7, lanes
    // 2-3 their D; the group's arrays are padded, so a tail tile stays inside.
    int dq_row[NDQ], dq_c[NDQ];
#pragma unroll
    for (int i = 0; i < NDQ; ++i) {
        const int idx = 64 * (wave + NW * i) + lane;
        dq_row[i] = idx / C8;
        dq_c[i] = ((idx % C8) ^ swz<D>(dq_row[i])) * 8;
    }
    const int hgl = kvh;  // head group = the G query heads of this K/V head
    const int qh0 = hgl * G;
    const float *l_src = p.ws_l + ws_base(p, b, hgl);
    const float *d_src = p.ws_d + ws_base(p, b, hgl);
    // Tiles are fetched in order (t_lo, t_lo + 1, ...), so each lane keeps its
    // next row as (position, head in group) and steps it by BR rows per tile
    // instead of dividing by G every time.
    const int step_pos = BR / G, step_hd = BR - step_pos * G;
    int dpos[NDQ], dhd[NDQ];
#pragma unroll
    for (int i = 0; i < NDQ; ++i) {
        const int rho = t_lo * BR + dq_row[i];
        dpos[i] = rho / G;
        dhd[i] = rho - dpos[i] * G;
    }
    auto dma_tile = [&](int t, int slotn) {
        (void)t;  // the lanes' row state holds tile t
        unsigned char *base = ring + (slotn % NS) * SLOT;
#pragma unroll
        for (int i = 0; i < NDQ; ++i) {
            // rows past the end read the last row
            const bool in = dpos[i] < Lq;
            const int pos = in ? dpos[i] : Lq - 1, hd = in ? dhd[i] : G - 1;
            const int64_t off = ((int64_t)(q_tok0 + pos) * p.Hq + qh0 + hd) * D + dq_c[i];
            const uint32_t dst = lds_addr(base) + 1024 * (wave_u + NW * i);
            lds_dma16_u((const __bf16 *)p.q + off, dst);
            lds_dma16_u((const __bf16 *)p.dout + off, dst + TILE * 2);
            dhd[i] += step_hd;
            dpos[i] += step_pos;
            if (dhd[i] >= G) {
                dhd[i] -= G;
                ++dpos[i];
            }
        }
        // tiles past the last one (issued so that every step has the same
        // loads) re-read the last tile's L and D
        const int r8 = min(t, t_hi - 1) * BR + 8 * wave + 4 * (lane & 1);
        const float *src = (lane & 2) ? d_src + r8 : l_src + r8;
        if (lane < 4) lds_dma16_u(src, lds_addr(base + 2 * TILE * 2) + 64 * wave_u);
    };

    // Row-slice read (A operand, rows 0..31 of a tile, chunk 2 s + half) and
    // transposing read (A = X^T: in 16-lane group g, lane j reads row
    // 4 (g >> 1) + j / 4 (+ 8 for the second read) of a 16-row slot, columns
    // d0 + 4 (j % 4) .. +3 with d0 = 32 i + 16 (g & 1)).
    // The chunk index sits in offset bits 3.., above the 4-element half-chunk
    // bit and below the row, so k-step s of the row-slice read is offset
    // rs0 ^ 16 s and block i of the transposing read tr0 ^ 32 i. Rows r and
    // r + 8 (r < 8) differ in bit 3 and swz(r + 8) = swz(r) ^ 2 for both head
    // dims: the second transposing read is at (first ^ 16) + 8 D. The
    // per-step offsets are formed inside the tile loop from these two bases
    // (an XOR each) rather than held in registers.
    const int rs0 = col * D + ((half ^ swz<D>(col)) * 8);
    const int vj = lane & 15, vg = lane >> 4;
    const int tr_row = 4 * (vg >> 1) + (vj >> 2);
    const int tr0 = tr_row * D + (((2 * (vg & 1) + ((vj & 3) >> 1)) ^ swz<D>(tr_row)) * 8) +
                    4 * (vj & 1);

    const float c = p.scale_log2;
    f32x16 dkacc[DBLK], dvacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) {
        dkacc[i] = f32x16{};
        dvacc[i] = f32x16{};
    }

    // Does every row of tile t exist and see every key of this wave (no
    // element mask needed)? Keys past the end are not masked: a lane's key
    // only reaches its own column of dK^T and dV^T, and the columns of keys
    // past the end are never stored.
    auto tile_full = [&](int t) {
        if (t * BR + BR > rows_total) return false;
        if (!CAUSAL) return true;
        return (t * BR) / G + shift >= wk1;
    };

    if constexpr (PIPE) {
        // S = Q K^T and dP = dO V^T of the tile in ring slot bs (rows 8 (j/4)
        // + 4 half + j%4, key col)
        auto scores = [&](const unsigned char *bs, int rs, f32x16 &sa, f32x16 &da) {
            const __bf16 *q_ = (const __bf16 *)bs;
            const __bf16 *g_ = (const __bf16 *)(bs + TILE * 2);
            bf16x8 qa[DSTEPS], ga[DSTEPS];
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s) {
                qa[s] = *(const bf16x8 *)(q_ + (rs ^ (16 * s)));
                ga[s] = *(const bf16x8 *)(g_ + (rs ^ (16 * s)));
            }
            sa = f32x16{};
            da = f32x16{};
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf[s], sa, 0, 0, 0);
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s) da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[s], vf[s], da, 0, 0, 0);
        };
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
        if (t_lo < t_hi) {
            for (int j = 0; j < NS - 1; ++j) dma_tile(t_lo + j, j);
            wait_barrier<(NS - 2) * NLOAD>();  // tile t_lo has landed
            int rs_b = rs0;
            asm volatile("" : "+v"(rs_b));
            scores(ring, rs_b, sacc, dpacc);
        }
        for (int t = t_lo; t < t_hi; ++t) {
            const int it = t - t_lo;
            // tile t + 1 has landed (tile t + 2 may not); every wave is done
            // with tile t - 1, whose slot the next DMA fills
            wait_barrier<(NS - 3) * NLOAD>();
            dma_tile(t + NS - 1, it + NS - 1);
            const unsigned char *base = ring + (it % NS) * SLOT;
            const unsigned char *nbase = ring + ((it + 1) % NS) * SLOT;
            int rs_b = rs0, tr_b = tr0;
            asm volatile("" : "+v"(rs_b), "+v"(tr_b));  // keep the derived offsets in the loop
            const __bf16 *qt = (const __bf16 *)base;
            const __bf16 *gt = (const __bf16 *)(base + TILE * 2);
            const float *misc = (const float *)(base + 2 * TILE * 2);
            bf16x8 tg[2][DBLK], tq[2][DBLK];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < DBLK; ++i) {
                    const int tri = tr_b ^ (32 * i);
                    const int o = 16 * h2 * D + tri, o8 = 16 * h2 * D + (tri ^ 16) + 8 * D;
                    const u32x2 g0 = lds_read_tr16(gt + o), g1 = lds_read_tr16(gt + o8);
                    const u32x2 q0 = lds_read_tr16(qt + o), q1 = lds_read_tr16(qt + o8);
                    tg[h2][i] = __builtin_bit_cast(bf16x8, u32x4{g0[0], g0[1], g1[0], g1[1]});
                    tq[h2][i] = __builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]});
                }
            float pv[16], dsv[16];
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const f32x4 lv = *(const f32x4 *)(misc + 16 * blk + 4 * half);
                const f32x4 dv4 = *(const f32x4 *)(misc + 16 * blk + 8 + 4 * half);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * blk + e;
                    pv[j] = fast_exp2(fmaf(sacc[j], c, -lv[e]));
                    dsv[j] = pv[j] * (dpacc[j] - dv4[e]);
                }
            }
            // the next tile's scores (the last step scores the re-loaded
            // tile past the end, which has landed too, and drops them)
            f32x16 sacc_n, dpacc_n;
            scores(nbase, rs_b, sacc_n, dpacc_n);
            if (!tile_full(t)) {
                // rows past the end carry arbitrary L and D: select, not scale
                const int rho0 = t * BR + 4 * half;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int rho = rho0 + 8 * (j >> 2) + (j & 3);
                    const bool vis = rho < rows_total && (!CAUSAL || rho >= row_min);
                    pv[j] = vis ? pv[j] : 0.f;
                    dsv[j] = vis ? dsv[j] : 0.f;
                }
            }
            bf16x8 pf[2], dsf[2];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                pf[j >> 3][j & 7] = (__bf16)pv[j];
                dsf[j >> 3][j & 7] = (__bf16)dsv[j];
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < DBLK; ++i) {
                    dvacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tg[h2][i], pf[h2], dvacc[i], 0, 0, 0);
                    dkacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[h2][i], dsf[h2], dkacc[i], 0, 0, 0);
                }
            sacc = sacc_n;
            dpacc = dpacc_n;
        }
    } else {
    // NS - 1 tiles in flight ahead of the one being computed.
    if (t_lo < t_hi)
        for (int j = 0; j < NS - 1; ++j) dma_tile(t_lo + j, j);
    for (int t = t_lo; t < t_hi; ++t) {
        const int it = t - t_lo;
        wait_barrier<(NS - 2) * NLOAD>();  // tile t has landed; every wave is done with tile t-1
        dma_tile(t + NS - 1, it + NS - 1);
        // Every wave runs every tile of the range (one path, no per-wave
        // skip): under a causal mask a tile wholly above this wave's keys
        // is masked to P = dS = 0.
        const unsigned char *base = ring + (it % NS) * SLOT;
        int rs_b = rs0, tr_b = tr0;
        asm volatile("" : "+v"(rs_b), "+v"(tr_b));  // keep the derived offsets in the loop
        const __bf16 *qt = (const __bf16 *)base;
        const __bf16 *gt = (const __bf16 *)(base + TILE * 2);
        const float *misc = (const float *)(base + 2 * TILE * 2);

        // S = Q K^T and dP = dO V^T: rows 8 (j/4) + 4 half + j%4, key col.
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
        // ONE: the tile's transposed operands (A of dV^T and dK^T), read
        // ahead of the exponentials
        bf16x8 tg[ONE ? 2 : 1][ONE ? DBLK : 1], tq[ONE ? 2 : 1][ONE ? DBLK : 1];
        if constexpr (ONE) {
            bf16x8 qa[DSTEPS], ga[DSTEPS];
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s) {
                qa[s] = *(const bf16x8 *)(qt + (rs_b ^ (16 * s)));
                ga[s] = *(const bf16x8 *)(gt + (rs_b ^ (16 * s)));
            }
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s)
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf[s], sacc, 0, 0, 0);
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s)
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[s], vf[s], dpacc, 0, 0, 0);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < DBLK; ++i) {
                    const int tri = tr_b ^ (32 * i);
                    const int o = 16 * h2 * D + tri, o8 = 16 * h2 * D + (tri ^ 16) + 8 * D;
                    const u32x2 g0 = lds_read_tr16(gt + o), g1 = lds_read_tr16(gt + o8);
                    const u32x2 q0 = lds_read_tr16(qt + o), q1 = lds_read_tr16(qt + o8);
                    tg[h2][i] = __builtin_bit_cast(bf16x8, u32x4{g0[0], g0[1], g1[0], g1[1]});
                    tq[h2][i] = __builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]});
                }
            // Issue order: the row slices of both products, then each product
            // MFMA followed by a share of the remaining reads (transposed
            // operands, then L and D), so that one wave keeps the LDS busy
            // while its matrix core runs.
            constexpr int NTR = 2 * 2 * DBLK * 2 + 8;  // transposing reads + L/D reads
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * DSTEPS, 0);
#pragma unroll
            for (int g = 0; g < 2 * DSTEPS; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, (NTR + 2 * DSTEPS - 1) / (2 * DSTEPS), 0);
            }
        } else {
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) {
            const bf16x8 a = *(const bf16x8 *)(qt + (rs_b ^ (16 * s)));
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[s], sacc, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) {
            const bf16x8 a = *(const bf16x8 *)(gt + (rs_b ^ (16 * s)));
            bf16x8 bv;
            if constexpr (VLDS)
                bv = *(const bf16x8 *)(vw + (rs_b ^ (16 * s)));
            else
                bv = vf[s];
            dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, dpacc, 0, 0, 0);
        }
        }
        // P = 2^(s c - L), dS = P (dP - D); masked pairs and rows past the end
        // give P = 0. B operands for k-step h2: rows 16 h2 + 8 (e/4) + 4 half + e%4.
        float pv[16], dsv[16];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const f32x4 lv = *(const f32x4 *)(misc + 16 * blk + 4 * half);
            const f32x4 dv4 = *(const f32x4 *)(misc + 16 * blk + 8 + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * blk + e;
                pv[j] = fast_exp2(fmaf(sacc[j], c, -lv[e]));
                dsv[j] = pv[j] * (dpacc[j] - dv4[e]);
            }
        }
        if (!tile_full(t)) {
            // rows past the end carry arbitrary L and D: select, not scale
            const int rho0 = t * BR + 4 * half;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rho = rho0 + 8 * (j >> 2) + (j & 3);
                const bool vis = rho < rows_total && (!CAUSAL || rho >= row_min);
                pv[j] = vis ? pv[j] : 0.f;
                dsv[j] = vis ? dsv[j] : 0.f;
            }
        }
        bf16x8 pf[2], dsf[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            pf[j >> 3][j & 7] = (__bf16)pv[j];
            dsf[j >> 3][j & 7] = (__bf16)dsv[j];
        }
        // dV^T += dO^T P, dK^T += Q^T dS (A operands by transposing reads).
        if constexpr (ONE) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < DBLK; ++i) {
                    dvacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tg[h2][i], pf[h2], dvacc[i], 0, 0, 0);
                    dkacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[h2][i], dsf[h2], dkacc[i], 0, 0, 0);
                }
        } else
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < DBLK; ++i) {
                const int tri = tr_b ^ (32 * i);
                const int o = 16 * h2 * D + tri, o8 = 16 * h2 * D + (tri ^ 16) + 8 * D;
                const u32x2 g0 = lds_read_tr16(gt + o), g1 = lds_read_tr16(gt + o8);
                const u32x2 q0 = lds_read_tr16(qt + o), q1 = lds_read_tr16(qt + o8);
                const bf16x8 ag = __builtin_bit_cast(bf16x8, u32x4{g0[0], g0[1], g1[0], g1[1]});
                const bf16x8 aq = __builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]});
                dvacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, pf[h2], dvacc[i], 0, 0, 0);
                dkacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, dsf[h2], dkacc[i], 0, 0, 0);
            }
    }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the (unused) tail loads

    // ---- write dK = scale dK^T^T and dV: lane owns key kk, head_dim
    // elements 32 i + 8 g + 4 half .. +3 (or this chunk's fp32 partials) ----
    if (!key_ok) continue;
    if (n_valid > 1) {
        float *pk = p.ws_part + ((int64_t)(grp * p.n_kb + kblk) * p.n_ch + chunk) * (2 * 128 * D) +
                    (32 * wave + col) * D + 4 * half;
        float *pv = pk + 128 * D;
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 wk, wv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wk[e] = dkacc[i][4 * g + e];
                    wv[e] = dvacc[i][4 * g + e];
                }
                *(f32x4 *)(pk + i * 32 + 8 * g) = wk;
                *(f32x4 *)(pv + i * 32 + 8 * g) = wv;
            }
        continue;
    }
    const int64_t off = ((int64_t)(k_tok0 + kk) * p.Hkv + kvh) * D + 4 * half;
    __bf16 *dkrow = (__bf16 *)p.dk + off;
    __bf16 *dvrow = (__bf16 *)p.dv + off;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 wk, wv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wk[e] = (__bf16)(dkacc[i][4 * g + e] * p.scale);
                wv[e] = (__bf16)dvacc[i][4 * g + e];
            }
            *(u32x2 *)(dkrow + i * 32 + 8 * g) = __builtin_bit_cast(u32x2, wk);
            *(u32x2 *)(dvrow + i * 32 + 8 * g) = __builtin_bit_cast(u32x2, wv);
        }
    }  // pass
}

// ---------------------------------------------------------------------------
// Sum of the row chunks' partial dK/dV for key blocks split into more than one
// chunk, in chunk order (deterministic): one workgroup per (sequence, K/V
// head, key block), four consecutive elements per thread and step.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(BwdParams p) {
    const int pid = blockIdx.x;  // (b * Hkv + kvh) * n_kb + key block
    const int grp = pid / p.n_kb, kblk = pid - grp * p.n_kb;
    const int b = grp / p.Hkv, kvh = grp - b * p.Hkv;
    const KeyBlockRows kr = key_block_rows<CAUSAL, VARLEN>(p, b, kblk);
    const int k0 = kblk * 128;
    if (k0 >= kr.Lk) return;
    const int n_valid = key_block_chunks(p, kr);
    if (n_valid <= 1) return;  // written directly by its only chunk
    const float *part = p.ws_part + (int64_t)pid * p.n_ch * (2 * 128 * D);
    constexpr int Q4 = D / 4;  // 4-element groups per key row
    for (int idx = threadIdx.x; idx < 128 * Q4; idx += 256) {
        const int key = idx / Q4, c4 = (idx - key * Q4) * 4;
        if (k0 + key >= kr.Lk) continue;
        f32x4 sk = f32x4{}, sv = f32x4{};
        for (int c = 0; c < n_valid; ++c) {
            const float *pc = part + (int64_t)c * (2 * 128 * D) + key * D + c4;
            sk += *(const f32x4 *)pc;
            sv += *(const f32x4 *)(pc + 128 * D);
        }
        const int64_t off = ((int64_t)(kr.k_tok0 + k0 + key) * p.Hkv + kvh) * D + c4;
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wk[e] = (__bf16)(sk[e] * p.scale);
            wv[e] = (__bf16)sv[e];
        }
        *(u32x2 *)((__bf16 *)p.dk + off) = __builtin_bit_cast(u32x2, wk);
        *(u32x2 *)((__bf16 *)p.dv + off) = __builtin_bit_cast(u32x2, wv);
    }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup owns 128 packed rows and walks the key tiles.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2))) void
bwd_dq_kernel(BwdParams p) {
    constexpr int BM = 32 * NW;            // packed rows per workgroup
    // keys per tile; at d = 64, 32 keys (144 VGPRs, 3 waves/SIMD) measured
    // 1-3 % faster than 64 keys (188 VGPRs, 2 waves/SIMD)
    constexpr int BN = 32;
    constexpr int KB = BN / 32;
    constexpr int C8 = D / 8;
    constexpr int DSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int TILE = BN * D;
    constexpr int NDK = TILE * 2 / 1024 / NW;  // loads per wave per K (or V) tile
    static_assert(NDK >= 1, "tile too small for one load per wave");
    constexpr int NLOAD = 2 * NDK;
    __shared__ __attribute__((aligned(1024))) __bf16 ring[NSLOT * 2 * TILE];

    const int tid = threadIdx.x;
    // wave-uniform wave index (scalar register)
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    // ---- workgroup -> (head group, row tile), as the forward ----
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
    const int kvh = hg % p.Hkv;
    int b = hg / p.Hkv;
    if constexpr (VARLEN) {
        if (p.B > 1 && p.B <= kLptMax) b = lpt_sequence(p.cu_q, p.cu_k, p.B, b, tid);  // longest first
    }
    const int G = p.G, qh0 = kvh * G;
    int q_tok0 = b * p.Sq, Lq = p.Sq, k_tok0 = b * p.Sk, Lk = p.Sk;
    if (VARLEN) {
        q_tok0 = p.cu_q[b];
        Lq = p.cu_q[b + 1] - q_tok0;
        k_tok0 = p.cu_k[b];
        Lk = p.cu_k[b + 1] - k_tok0;
    }
    const int rows_total = Lq * G;
    const int row0 = rb * BM;
    if (row0 >= rows_total) return;  // uniform over the workgroup
    const int shift = Lk - Lq;
    int kend = Lk;
    if (CAUSAL) {
        const int last = min(row0 + BM, rows_total) - 1;
        kend = min(Lk, last / G + 1 + shift);
    }
    const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

    // ---- this lane's query row ----
    const int rho = row0 + wave * 32 + col;
    const bool row_ok = rho < rows_total;
    const int pos = rho / G;
    const int head = qh0 + (rho - pos * G);
    const int row_kend = CAUSAL ? min(Lk, pos + 1 + shift) : Lk;
    // Every wave runs every key tile of the workgroup (one path, no per-wave
    // skip); keys past a row's causal limit are masked to P = 0, and rows
    // past the end have L = +inf (P = 0) and are never stored.
    const int wave_kfull = CAUSAL ? min(Lk, (row0 + wave * 32) / G + 1 + shift) : Lk;

    // Per-row statistics and the Q^T / dO^T fragments (B operands). This
    // pass also forms the row statistics for the key-block pass that follows
    // it: D = rowsum(dO * O) (the lane's half of the row, then its partner
    // lane's) and L in log2 units (+inf for a row that sees no key, so that
    // P = 0 there), stored in packed-row order.
    float lrow = INFINITY, drow = 0.f;
    bf16x8 qf[DSTEPS], gf[DSTEPS];
    {
        const int qpos = row_ok ? pos : Lq - 1;
        const int qhead = row_ok ? head : qh0;
        const int64_t off = ((int64_t)(q_tok0 + qpos) * p.Hq + qhead) * D + 8 * half;
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) {
            const u32x4 a = *(const u32x4 *)((const __bf16 *)p.q + off + 16 * s);
            const u32x4 g2 = *(const u32x4 *)((const __bf16 *)p.dout + off + 16 * s);
            const u32x4 o2 = *(const u32x4 *)((const __bf16 *)p.o + off + 16 * s);
            qf[s] = __builtin_bit_cast(bf16x8, row_ok ? a : u32x4{0u, 0u, 0u, 0u});
            gf[s] = __builtin_bit_cast(bf16x8, row_ok ? g2 : u32x4{0u, 0u, 0u, 0u});
            const bf16x8 o8 = __builtin_bit_cast(bf16x8, o2);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)o8[e], (float)gf[s][e], acc);
        }
        drow = pair_sum32(acc);
        if (row_ok) {
            const int64_t li = VARLEN ? (int64_t)(q_tok0 + pos) * p.Hq + head
                                      : ((int64_t)b * p.Hq + head) * p.Sq + pos;
            const float l = p.lse[li];
            lrow = l == -INFINITY ? INFINITY : l * kLog2e;
            if (half == 0) {
                const int64_t wi = ws_base(p, b, kvh) + rho;
                p.ws_d[wi] = drow;
                p.ws_l[wi] = lrow;
            }
        }
        u32x4 x = __builtin_bit_cast(u32x4, qf[0]) ^ __builtin_bit_cast(u32x4, gf[0]);
#pragma unroll
        for (int s = 1; s < DSTEPS; ++s)
            x ^= __builtin_bit_cast(u32x4, qf[s]) ^ __builtin_bit_cast(u32x4, gf[s]);
        const uint32_t y = x[0] ^ x[1] ^ x[2] ^ x[3] ^ __builtin_bit_cast(uint32_t, lrow) ^
                           __builtin_bit_cast(uint32_t, drow);
        asm volatile("" ::"v"(y));
    }

    // ---- DMA of key tile t of K and V into a ring slot ----
    int dk_row[NDK], dk_c[NDK];
#pragma unroll
    for (int i = 0; i < NDK; ++i) {
        const int idx = 64 * (wave + NW * i) + lane;
        dk_row[i] = idx / C8;
        dk_c[i] = ((idx % C8) ^ swz<D>(dk_row[i])) * 8;
    }
    // A key tile is addressed as a wave-uniform base (scalar registers) plus
    // 24-bit per-lane byte offsets; rows past kend read the last needed key
    // and tiles past the end re-load the last needed tile.
    const int64_t kv_stride = (int64_t)p.Hkv * D;
    const char *kbase = (const char *)((const __bf16 *)p.k + ((int64_t)k_tok0 * p.Hkv + kvh) * D);
    const char *vbase = (const char *)((const __bf16 *)p.v + ((int64_t)k_tok0 * p.Hkv + kvh) * D);
    const uint32_t row_bytes = (uint32_t)kv_stride * 2;  // < 2^24 (Hkv d <= 2^22)
    const uint32_t tile_bytes = BN * row_bytes;
    auto dma_tile = [&](int t, int slotn) {
        __bf16 *kd = ring + slotn * 2 * TILE;
        const int tt = min(t, ntiles - 1);
        const int last = kend - 1 - tt * BN;  // last needed row of the tile (>= 0)
        const uint64_t toff = (uint64_t)(uint32_t)tt * tile_bytes;
#pragma unroll
        for (int i = 0; i < NDK; ++i) {
            const uint32_t voff = __umul24((uint32_t)min(dk_row[i], last), row_bytes) + dk_c[i] * 2;
            const uint32_t dst =
                (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds_addr(kd) + 1024 * (wave + NW * i)));
            lds_dma16_sv(uniform_ptr(kbase + toff), voff, dst);
            lds_dma16_sv(uniform_ptr(vbase + toff), voff, dst + TILE * 2);
        }
    };

    int rs_rd[DSTEPS];
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) rs_rd[s] = col * D + (((2 * s + half) ^ swz<D>(col)) * 8);
    // The swizzle depends on row bits 0..3, so the second read (row + 8) has
    // its own offset; +16 and +32 rows keep the swizzle.
    const int vj = lane & 15, vg = lane >> 4;
    const int tr_row = 4 * (vg >> 1) + (vj >> 2);
    int tr_rd[DBLK], tr_rd8[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) {
        const int chunk = 4 * i + 2 * (vg & 1) + ((vj & 3) >> 1);
        tr_rd[i] = tr_row * D + ((chunk ^ swz<D>(tr_row)) * 8) + 4 * (vj & 1);
        tr_rd8[i] = (tr_row + 8) * D + ((chunk ^ swz<D>(tr_row + 8)) * 8) + 4 * (vj & 1);
    }

    const float c = p.scale_log2;
    f32x16 dqacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) dqacc[i] = f32x16{};

    if (ntiles > 0) {
        dma_tile(0, 0);
        dma_tile(1, 1);
    }
    for (int t = 0; t < ntiles; ++t) {
        wait_barrier<NLOAD>();  // tile t has landed; every wave is done with tile t-1
        dma_tile(t + 2, (t + 2) % NSLOT);
        const __bf16 *kt = ring + (t % NSLOT) * 2 * TILE;
        const __bf16 *vt = kt + TILE;
        // S^T = K Q^T, dP^T = V dO^T: keys kb*32 + 8 (j/4) + 4 half + j%4, row col.
        f32x16 sacc[KB], dpacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sacc[kb] = f32x16{};
            dpacc[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s) {
                const bf16x8 a = *(const bf16x8 *)(kt + kb * 32 * D + rs_rd[s]);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < DSTEPS; ++s) {
                const bf16x8 a = *(const bf16x8 *)(vt + kb * 32 * D + rs_rd[s]);
                dpacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[s], dpacc[kb], 0, 0, 0);
            }
        }
        // dS^T = P^T (dP^T - D), P^T = 2^(s c - L); masked keys give P = 0.
        float pv[KB][16];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) pv[kb][j] = fast_exp2(fmaf(sacc[kb][j], c, -lrow));
        if ((t + 1) * BN > wave_kfull) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = t * BN + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
                    pv[kb][j] = key < row_kend ? pv[kb][j] : 0.f;
                }
        }
        bf16x8 dsf[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                dsf[kb][j >> 3][j & 7] = (__bf16)(pv[kb][j] * (dpacc[kb][j] - drow));
        // dQ^T += K^T dS^T (A = K^T by transposing reads).
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < DBLK; ++i) {
                    const __bf16 *kp = kt + (kb * 32 + 16 * h2) * D;
                    const u32x2 lo = lds_read_tr16(kp + tr_rd[i]), hi = lds_read_tr16(kp + tr_rd8[i]);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                    dqacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[kb][h2], dqacc[i], 0, 0, 0);
                }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- write dQ = scale dQ^T^T: lane owns row rho ----
    if (!row_ok) return;
    __bf16 *qrow = (__bf16 *)p.dq + ((int64_t)(q_tok0 + pos) * p.Hq + head) * D + 4 * half;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(dqacc[i][4 * g + e] * p.scale);
            *(u32x2 *)(qrow + i * 32 + 8 * g) = __builtin_bit_cast(u32x2, w);
        }
}

// Compute units of the current device (256 on MI355X).
int device_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const BwdParams &p, hipStream_t s) {
    // dQ first: it also writes the row statistics D and L that the key-block
    // pass reads.
    const long long q_grid = (long long)p.n_hg * p.n_rb;
    if (q_grid > 0) {
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)q_grid),
                           dim3(NTHREADS), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long kv_blocks = (long long)p.B * p.Hkv * p.n_kb;
    if (kv_blocks > 0) {
        // Under a causal mask key block i sees far more rows than the last
        // ones: pair block i with n_kb - 1 - i in one workgroup so that the
        // workgroups are about equally long (unless the rows are chunked).
        BwdParams pk = p;
        pk.pair = CAUSAL && p.n_ch == 1;
        const long long grid = pk.pair ? (long long)p.B * p.Hkv * ((p.n_kb + 1) / 2)
                                       : kv_blocks * p.n_ch;
        // A grid of at most one workgroup per CU runs one wave per SIMD
        // whatever the register budget: take the variant built for that.
        if (D == 128 && grid <= device_cu_count())
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN, D == 128>), dim3((unsigned)grid),
                               dim3(NTHREADS), 0, s, pk);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN, false>), dim3((unsigned)grid),
                               dim3(NTHREADS), 0, s, pk);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.n_ch > 1) {
            hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<D, CAUSAL, VARLEN>),
                               dim3((unsigned)kv_blocks), dim3(256), 0, s, p);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

int bwd_rows_per_tile() { return 32 * NW; }

hipError_t launch_bwd_bf16(const BwdParams &p, int d, bool causal, bool varlen, hipStream_t s) {
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
