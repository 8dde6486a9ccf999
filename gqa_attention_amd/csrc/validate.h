// Host-side argument checks for the C ABI. Plain C++ with no HIP dependency:
// every check runs before anything touches the GPU, so every error path can be
// exercised on a machine without one.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "gqa_attn.h"

namespace gqa {

constexpr int kMaxSplits = 64;
constexpr int kSplitAlign = 64;  // split chunk granularity (keys)
constexpr int kBwdPadFloats = 128;  // spare floats after each backward statistics array

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline bool supported_d(int d) { return d == 64 || d == 128; }

inline int check_common(int dtype, int d, float scale) {
    if (dtype != GQA_DTYPE_BF16 && dtype != GQA_DTYPE_FP32) return GQA_EUNSUPPORTED;
    if (!supported_d(d)) return GQA_EUNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_EINVAL;
    return GQA_OK;
}

inline int validate_fwd(const void *q, const void *k, const void *v, const void *out,
                        const float *lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                        float scale, const int32_t *cu_q, const int32_t *cu_k, int dtype) {
    if (!q || !k || !v || !out || !lse) return GQA_EINVAL;
    const int rc = check_common(dtype, d, scale);
    if (rc != GQA_OK) return rc;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return GQA_EINVAL;
    const bool varlen = cu_q != nullptr;
    if ((cu_q == nullptr) != (cu_k == nullptr)) return GQA_EINVAL;
    if (varlen) {
        if (Sq < 0 || Sk < 0) return GQA_EINVAL;
        if (!aligned(cu_q, 4) || !aligned(cu_k, 4)) return GQA_EINVAL;
    } else if (Sq < 1 || Sk < 1) {
        return GQA_EINVAL;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(lse, 4))
        return GQA_EINVAL;
    // K/V row pitch: the forward kernel addresses a key tile with 24-bit
    // per-lane byte offsets (row pitch 2 Hkv d bytes < 2^24).
    if ((long long)Hkv * d > (1LL << 22)) return GQA_EINVAL;
    // Launch grid: head groups x row tiles must fit a 1-D grid (<= 2^31 - 1).
    const long long tiles = ((long long)Hq * Sq + 31) / 32;
    if ((long long)B * tiles > 0x7fffffffLL) return GQA_EINVAL;
    return GQA_OK;
}

// Decode workspace (num_splits > 1): fp32 partial outputs [ns, B*Hq, d]
// (the size rounded up to 256 bytes), then fp32 partial LSEs [ns, B*Hq].
inline size_t decode_workspace_o_bytes(int B, int Hq, int d, int num_splits) {
    return ((size_t)B * Hq * num_splits * d * sizeof(float) + 255) & ~size_t(255);
}
inline size_t decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
    if (B < 1 || Hq < 1 || !supported_d(d) || num_splits < 1 || num_splits > kMaxSplits) return 0;
    if (num_splits == 1) return 0;
    return decode_workspace_o_bytes(B, Hq, d, num_splits) + (size_t)B * Hq * num_splits * sizeof(float);
}

inline int split_chunk(int Sk, int num_splits) {
    const long long chunk = ((long long)Sk + num_splits - 1) / num_splits;
    const long long aligned_chunk = (chunk + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
    return (int)(aligned_chunk < 0x7fffffc0LL ? aligned_chunk : 0x7fffffc0LL);
}

inline int validate_decode(const void *q, const void *kc, const void *vc, const void *out,
                           const float *lse, int B, int Hq, int Hkv, int Sk, int d, float scale,
                           int num_splits, const void *ws, size_t ws_bytes, int dtype) {
    if (!q || !kc || !vc || !out || !lse) return GQA_EINVAL;
    const int rc = check_common(dtype, d, scale);
    if (rc != GQA_OK) return rc;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sk < 1 || Hq % Hkv != 0) return GQA_EINVAL;
    if (num_splits < 1 || num_splits > kMaxSplits) return GQA_EINVAL;
    if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 16) ||
        !aligned(lse, 4))
        return GQA_EINVAL;
    if ((long long)B * Hkv * num_splits * ((Hq / Hkv + 15) / 16) > 0x7fffffffLL) return GQA_EINVAL;
    if (num_splits > 1) {
        if (!ws || !aligned(ws, 16)) return GQA_EWORKSPACE;
        if (ws_bytes < decode_workspace_bytes(B, Hq, d, num_splits)) return GQA_EWORKSPACE;
    }
    return GQA_OK;
}

// Row statistics of the backward: 2 arrays of B * Hq * R floats (R = Sq * G
// rounded up to 4 per head group) plus kBwdPad floats each.
inline size_t bwd_workspace_floats(int B, int Hq, int Hkv, int Sq) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 0) return 0;
    const long long G = Hq / Hkv;
    const long long rows = (long long)B * Hkv * (((long long)Sq * G + 3) & ~3LL);
    return (size_t)(rows + kBwdPadFloats);
}
// Backward row chunks. The dK/dV pass has one workgroup per (sequence, K/V
// head, 128-key block); when there are fewer than kBwdMinBlocks of those (a
// single sequence with few K/V heads) the rows that see each key block are
// split into up to n_ch chunks of ch_tiles 32-row tiles (at least
// kBwdMinChunkTiles), aiming at kBwdTargetWgs workgroups, and the chunks' fp32
// partial dK/dV are summed afterwards. Sized for 256 CUs.
constexpr int kBwdMinBlocks = 256, kBwdTargetWgs = 512, kBwdMinChunkTiles = 32;
struct BwdChunks {
    int n_ch, ch_tiles;
};
inline BwdChunks bwd_chunks(int B, int Hq, int Hkv, int Sq, int Sk) {
    BwdChunks c{1, 1 << 30};
    if (B < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 1 || Sk < 1) return c;
    const long long blocks = (long long)B * Hkv * ((Sk + 127) / 128);
    if (blocks >= kBwdMinBlocks) return c;
    const long long tiles = ((long long)Sq * (Hq / Hkv) + 31) / 32;  // most per key block
    long long n = (kBwdTargetWgs + blocks - 1) / blocks;
    n = n < tiles / kBwdMinChunkTiles ? n : tiles / kBwdMinChunkTiles;
    if (n <= 1) return c;
    c.n_ch = (int)n;
    c.ch_tiles = (int)((tiles + n - 1) / n);
    return c;
}
// Floats of partial dK/dV: per (sequence, K/V head, key block, chunk) 2 x 128 x d.
inline size_t bwd_partial_floats(int B, int Hq, int Hkv, int Sq, int Sk, int d) {
    const int nch = bwd_chunks(B, Hq, Hkv, Sq, Sk).n_ch;
    if (nch <= 1) return 0;
    const long long n_kb = (Sk + 127) / 128;
    return (size_t)((long long)B * Hkv * n_kb * nch * 2 * 128 * d);
}
inline size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d) {
    const size_t n = bwd_workspace_floats(B, Hq, Hkv, Sq);
    if (!n || Sk < 0 || (d != 64 && d != 128)) return 0;
    return (2 * n + bwd_partial_floats(B, Hq, Hkv, Sq, Sk, d)) * sizeof(float);
}

inline int validate_bwd(const void *q, const void *k, const void *v, const void *out,
                        const float *lse, const void *dout, const void *dq, const void *dk,
                        const void *dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale,
                        const int32_t *cu_q, const int32_t *cu_k, const void *ws,
                        size_t ws_bytes, int dtype) {
    const int rc = validate_fwd(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, d, scale, cu_q, cu_k, dtype);
    if (rc != GQA_OK) return rc;
    if (dtype != GQA_DTYPE_BF16) return GQA_EUNSUPPORTED;
    if (!dout || !dq || !dk || !dv) return GQA_EINVAL;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return GQA_EINVAL;
    if (!ws || !aligned(ws, 16) || ws_bytes < bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d))
        return GQA_EWORKSPACE;
    return GQA_OK;
}

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// A per-tensor dequantisation scale: finite and > 0.
inline bool valid_dequant_scale(float s) { return std::isfinite(s) && s > 0.f; }

inline int validate_decode_ex(const void *q, const void *kc, const void *vc, const void *out,
                              const float *lse, int B, int Hq, int Hkv, int d, float scale,
                              const int32_t *seqlens, int max_seqlen_k, const int32_t *table,
                              int block_size, int max_blocks, int window_left, int kv_dtype,
                              float k_scale, float v_scale, int num_splits, const void *ws,
                              size_t ws_bytes) {
    if (!q || !kc || !vc || !out || !lse) return GQA_EINVAL;
    if (kv_dtype != GQA_DTYPE_BF16 && kv_dtype != GQA_DTYPE_FP8_E4M3) return GQA_EUNSUPPORTED;
    if (!supported_d(d)) return GQA_EUNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_EINVAL;
    if (kv_dtype == GQA_DTYPE_FP8_E4M3 &&
        (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) || !(v_scale > 0.f)))
        return GQA_EINVAL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_seqlen_k < 1) return GQA_EINVAL;
    if (window_left < -1) return GQA_EINVAL;
    if (num_splits < 1 || num_splits > kMaxSplits) return GQA_EINVAL;
    if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 16) ||
        !aligned(lse, 4) || (seqlens && !aligned(seqlens, 4)))
        return GQA_EINVAL;
    if (table) {
        if (!aligned(table, 4) || !is_pow2(block_size) || block_size > 4096) return GQA_EINVAL;
        if ((long long)max_blocks * block_size < max_seqlen_k) return GQA_EINVAL;
    }
    if ((long long)B * Hkv * num_splits * ((Hq / Hkv + 15) / 16) > 0x7fffffffLL) return GQA_EINVAL;
    if (num_splits > 1) {
        if (!ws || !aligned(ws, 16)) return GQA_EWORKSPACE;
        if (ws_bytes < decode_workspace_bytes(B, Hq, d, num_splits)) return GQA_EWORKSPACE;
    }
    return GQA_OK;
}

// Split count for decode (measured on MI355X): enough splits that the launch
// has about 192 or more workgroups (at least 2 for ragged batches), but at
// least 512 keys per split.
inline int decode_num_splits(int B, int Hq, int Hkv, int d, int max_seqlen_k, int window_left,
                             bool ragged) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || !supported_d(d) || max_seqlen_k < 1 ||
        window_left < -1)
        return 0;
    const long long units = (long long)B * Hkv * ((Hq / Hkv + 15) / 16);
    int ns = units >= 192 ? 1 : units >= 96 ? 2 : units >= 48 ? 4 : units >= 12 ? 8 : 16;
    // a window of at most half the longest length caps most visible ranges
    // at the same length, so the batch is no longer ragged in what it reads
    const bool window_evens = window_left >= 0 && 2LL * (window_left + 1) <= max_seqlen_k;
    if (ragged && !window_evens && ns < 2) ns = 2;
    const long long keys = window_left >= 0 && (long long)window_left + 1 < max_seqlen_k
                               ? (long long)window_left + 1
                               : max_seqlen_k;
    while (ns > 1 && keys / ns < 512) ns >>= 1;
    return ns;
}

}  // namespace gqa
