// Launch parameters shared by the host launchers and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gqa {

// One forward launch (prefill / encoder). A "head group" is the set of query
// heads one workgroup packs into its row tile: the G = Hq / Hkv heads that
// share a K/V head (pack_gqa) or a single query head when packing is off.
struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const int32_t *cu_q, *cu_k;  // both null for fixed length
    int B, Hq, Hkv, Sq, Sk;      // Sq / Sk: lengths, or the maxima for variable length
    int G;                       // Hq / Hkv
    int gpack;                   // query heads per row tile: G or 1
    int n_hg;                    // B * Hq / gpack
    int n_rb;                    // row tiles per head group
    float scale;                 // softmax scale (> 0)
    float scale_log2;            // scale * log2(e) (* q_scale * k_scale for fp8 inputs)
    float o_scale;               // fp8 inputs: V dequantisation scale applied to O (else 1)
    // split-KV partial mode (fp32 kernel only, Sq == 1): key range of split s
    // is [s * split_chunk, (s + 1) * split_chunk); partials go to ws_o / ws_lse.
    int num_splits;
    int split_chunk;
    float *ws_o;
    float *ws_lse;
    // bf16 / fp8 kernel scheduling: 0 one row tile per workgroup; 1
    // persistent, tiles claimed through the counters at sched (nine unsigned
    // ints, zero on entry and on exit)
    int persist;
    unsigned int *sched;
    // bf16 / fp8 kernels: divisions by launch constants as multiply-high and
    // shift (fastdiv.h): by gpack, by G, by hpb = Hq / gpack (head groups per
    // sequence) and by n_rb; set by the launcher
    int hpb;
    unsigned int gp_m, g_m, hpb_m, rb_m;
    int gp_sh, g_sh, hpb_sh, rb_sh;
};

// One split-KV decode launch (bf16 queries; bf16 or fp8 e4m3 K/V cache).
struct DecodeParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, Hq, Hkv, Sk, G;       // Sk: keys per sequence, or the maximum when seqlens is set
    int n_qs;                    // query slices of 16 heads per K/V head: ceil(G / 16)
    int num_splits;
    float scale_log2;            // scale * log2(e) (* k dequantisation scale for fp8)
    float v_scale;               // V dequantisation scale (1 for bf16)
    const int32_t *seqlens;      // [B] keys per sequence, or null (all Sk)
    const int32_t *block_table;  // [B, max_blocks] page of each block of block_size keys, or null
    int log2_block;              // log2(block_size) when paged
    int max_blocks;
    int window_left;             // -1: whole cache; W >= 0: keys j >= L - 1 - W
    float *ws_o;                 // [num_splits, B*Hq, d] fp32, used when num_splits > 1
    float *ws_lse;               // [num_splits, B*Hq] fp32
};

// One backward launch (three kernels: row statistics, dK/dV, dQ). The
// workspace holds two fp32 arrays in packed-row order: for sequence b and
// head group g (the G query heads of one K/V head), row rho = pos * G + r is
// element (b * (Hq / G) + g) * R + rho with R = Sq * G rounded up to a
// multiple of 4; each array is followed by 128 spare floats so that whole
// 32-row tiles (and the prefetch two tiles ahead) can be fetched.
struct BwdParams {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    const int32_t *cu_q, *cu_k;  // both null for fixed length
    int B, Hq, Hkv, Sq, Sk, G;   // Sq / Sk: lengths, or the maxima for variable length
    int n_hg;                    // B * Hkv head groups (dQ grid)
    int n_rb;                    // 128-row tiles per head group (dQ grid)
    int n_kb;                    // 128-key blocks per sequence (dK/dV grid)
    float scale, scale_log2;
    float *ws_d;                 // rowsum(dO * O)
    float *ws_l;                 // LSE in log2 units, +inf for rows that see no key
    // Row chunks (n_ch = 1: none): the rows that see a key block are split
    // into chunks of ch_tiles 32-row tiles, n_ch per key block at most (the
    // last runs to the end). A key block with more than one non-empty chunk
    // writes fp32 partials, [2][128 keys][d] per chunk at ws_part +
    // (((b * Hkv + kvh) * n_kb + key block) * n_ch + chunk) * 256 d, summed
    // into dK/dV by a reduction pass.
    int n_ch, ch_tiles;
    float *ws_part;
    // Paired key blocks (causal, n_ch = 1): a dK/dV workgroup takes key block
    // i and then n_kb(b) - 1 - i; the grid has (n_kb + 1) / 2 per head group.
    int pair;
};

// Launchers (one per kernel family). Each returns a hipError_t.
hipError_t launch_fwd_bf16(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams &p, int d, bool causal, bool varlen, bool split,
                          hipStream_t s);
hipError_t launch_decode_bf16(const DecodeParams &p, int d, bool paged, bool fp8_kv, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdParams &p, int d, bool causal, bool varlen, hipStream_t s);
hipError_t launch_decode_combine(const float *ws_o, const float *ws_lse, void *out, float *lse,
                                 int rows, int num_splits, int d, bool out_bf16, hipStream_t s);

}  // namespace gqa
