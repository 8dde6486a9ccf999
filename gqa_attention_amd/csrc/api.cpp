// C ABI entry points: validate on the host, pick the kernel instance and the
// grid, launch asynchronously on the caller's stream. Nothing here allocates,
// synchronises or reads device memory.

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include <hip/hip_runtime.h>

#include "gqa_attn.h"
#include "params.h"
#include "validate.h"

namespace gqa {
int fwd_bf16_rows_per_tile(int d);
int fwd_f32_rows_per_tile();
int bwd_rows_per_tile();
}  // namespace gqa

namespace {

// Debug knob for A/B measurements of query-head packing: GQA_ATTN_PACK=0
// gives every query head its own row tiles (K/V then re-read per head).
bool pack_enabled() {
    static const bool on = [] {
        const char *e = std::getenv("GQA_ATTN_PACK");
        return !(e && std::strcmp(e, "0") == 0);
    }();
    return on;
}

int status_from(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ELAUNCH; }

// Pointers into a decode workspace (num_splits > 1; both null otherwise).
void split_workspace(void *workspace, int B, int Hq, int d, int num_splits, float *&ws_o,
                     float *&ws_lse) {
    ws_o = nullptr;
    ws_lse = nullptr;
    if (num_splits <= 1) return;
    ws_o = static_cast<float *>(workspace);
    ws_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                       gqa::decode_workspace_o_bytes(B, Hq, d, num_splits));
}

// Static scratch of gqa_attn_decode_noalloc: the split partials of callers
// that cannot allocate. Every GPU the library runs on holds its own copy
// until the process ends. In host code the name `scratch` is only a stand-in
// for the symbol: its device address (different on every GPU) comes from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) unsigned char scratch[GQA_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or null if it cannot be
// obtained.
void *scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char *gqa_attn_strerror(int status) {
    switch (status) {
        case GQA_OK: return "success";
        case GQA_EINVAL: return "invalid argument";
        case GQA_EUNSUPPORTED: return "unsupported head_dim or dtype";
        case GQA_EWORKSPACE: return "decode workspace missing or too small";
        case GQA_ELAUNCH: return "kernel launch failed";
        case GQA_ESCRATCH: return "decode partials exceed the static scratch buffer";
        default: return "unknown status";
    }
}

int gqa_attn_decode_num_splits(int B, int Hq, int Hkv, int d, int max_seqlen_k, int window_left,
                               int ragged) {
    return gqa::decode_num_splits(B, Hq, Hkv, d, max_seqlen_k, window_left, ragged != 0);
}

size_t gqa_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d) {
    return gqa::bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d);
}

int gqa_attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Sq,
                 int Sk, int d, float scale, int causal, const int32_t *cu_seqlens_q,
                 const int32_t *cu_seqlens_k, void *workspace, size_t workspace_bytes, int dtype,
                 void *stream) {
    const int rc = gqa::validate_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d,
                                     scale, cu_seqlens_q, cu_seqlens_k, workspace,
                                     workspace_bytes, dtype);
    if (rc != GQA_OK) return rc;
    gqa::BwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = out;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sq = Sq;
    p.Sk = Sk;
    p.G = Hq / Hkv;
    p.n_hg = B * Hkv;
    const int rows = gqa::bwd_rows_per_tile();
    p.n_rb = (int)(((long long)p.G * Sq + rows - 1) / rows);
    p.n_kb = (Sk + 127) / 128;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    const size_t n = gqa::bwd_workspace_floats(B, Hq, Hkv, Sq);
    p.ws_d = static_cast<float *>(workspace);
    p.ws_l = p.ws_d + n;
    const gqa::BwdChunks ch = gqa::bwd_chunks(B, Hq, Hkv, Sq, Sk);
    p.n_ch = ch.n_ch;
    p.ch_tiles = ch.ch_tiles;
    p.ws_part = p.n_ch > 1 ? p.ws_l + n : nullptr;
    (void)hipGetLastError();
    return status_from(gqa::launch_bwd_bf16(p, d, causal != 0, cu_seqlens_q != nullptr,
                                            static_cast<hipStream_t>(stream)));
}

size_t gqa_attn_decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
    return gqa::decode_workspace_bytes(B, Hq, d, num_splits);
}

int gqa_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse, int B, int Hq,
                 int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int dtype,
                 void *stream) {
    const int rc = gqa::validate_fwd(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, d, scale,
                                     cu_seqlens_q, cu_seqlens_k, dtype);
    if (rc != GQA_OK) return rc;
    if (Sq == 0) return GQA_OK;  // variable length with no query rows at all

    const bool varlen = cu_seqlens_q != nullptr;
    gqa::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = out;
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sq = Sq;
    p.Sk = Sk;
    p.G = Hq / Hkv;
    p.gpack = pack_enabled() ? p.G : 1;
    p.n_hg = B * (Hq / p.gpack);
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.num_splits = 1;
    const int rows = dtype == GQA_DTYPE_BF16 ? gqa::fwd_bf16_rows_per_tile(d)
                                             : gqa::fwd_f32_rows_per_tile();
    p.n_rb = (int)(((long long)p.gpack * Sq + rows - 1) / rows);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (dtype == GQA_DTYPE_BF16)
        return status_from(gqa::launch_fwd_bf16(p, d, causal != 0, varlen, s));
    return status_from(gqa::launch_fwd_f32(p, d, causal != 0, varlen, false, s));
}

int gqa_attn_fwd_fp8(const void *q, const void *k, const void *v, void *out, float *lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, float q_scale,
                     float k_scale, float v_scale, void *stream) {
    // same geometry rules as the bf16 forward (one byte per element instead
    // of two only relaxes them)
    const int rc = gqa::validate_fwd(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, d, scale,
                                     cu_seqlens_q, cu_seqlens_k, GQA_DTYPE_BF16);
    if (rc != GQA_OK) return rc;
    if (!gqa::valid_dequant_scale(q_scale) || !gqa::valid_dequant_scale(k_scale) ||
        !gqa::valid_dequant_scale(v_scale))
        return GQA_EINVAL;
    const float c = scale * q_scale * k_scale * 1.4426950408889634f;
    if (!(c > 0.f) || !std::isfinite(c)) return GQA_EINVAL;
    if (Sq == 0) return GQA_OK;
    gqa::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = out;
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sq = Sq;
    p.Sk = Sk;
    p.G = Hq / Hkv;
    p.gpack = pack_enabled() ? p.G : 1;
    p.n_hg = B * (Hq / p.gpack);
    p.scale = scale;
    p.scale_log2 = c;
    p.o_scale = v_scale;
    p.num_splits = 1;
    const int rows = gqa::fwd_bf16_rows_per_tile(d);
    p.n_rb = (int)(((long long)p.gpack * Sq + rows - 1) / rows);
    (void)hipGetLastError();
    return status_from(gqa::launch_fwd_fp8(p, d, causal != 0, cu_seqlens_q != nullptr,
                                           static_cast<hipStream_t>(stream)));
}

int gqa_attn_decode(const void *q, const void *k_cache, const void *v_cache, void *out,
                    float *lse, int B, int Hq, int Hkv, int Sk, int d, float scale,
                    int num_splits, void *workspace, size_t workspace_bytes, int dtype,
                    void *stream) {
    const int rc = gqa::validate_decode(q, k_cache, v_cache, out, lse, B, Hq, Hkv, Sk, d, scale,
                                        num_splits, workspace, workspace_bytes, dtype);
    if (rc != GQA_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int chunk = gqa::split_chunk(Sk, num_splits);
    const int rows = B * Hq;
    float *ws_o = nullptr, *ws_lse = nullptr;
    split_workspace(workspace, B, Hq, d, num_splits, ws_o, ws_lse);
    (void)hipGetLastError();
    if (dtype == GQA_DTYPE_BF16) {
        gqa::DecodeParams p{};
        p.q = q;
        p.k = k_cache;
        p.v = v_cache;
        p.o = out;
        p.lse = lse;
        p.B = B;
        p.Hq = Hq;
        p.Hkv = Hkv;
        p.Sk = Sk;
        p.G = Hq / Hkv;
        p.n_qs = (p.G + 15) / 16;
        p.num_splits = num_splits;
        p.scale_log2 = scale * 1.4426950408889634f;
        p.v_scale = 1.f;
        p.seqlens = nullptr;
        p.block_table = nullptr;
        p.window_left = -1;
        p.ws_o = ws_o;
        p.ws_lse = ws_lse;
        hipError_t e = gqa::launch_decode_bf16(p, d, false, false, s);
        if (e != hipSuccess || num_splits == 1) return status_from(e);
        return status_from(
            gqa::launch_decode_combine(ws_o, ws_lse, out, lse, rows, num_splits, d, true, s));
    }
    // fp32: the fp32 forward kernel with one query position per sequence.
    gqa::FwdParams p{};
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.o = out;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sq = 1;
    p.Sk = Sk;
    p.G = Hq / Hkv;
    p.gpack = pack_enabled() ? p.G : 1;
    p.n_hg = B * (Hq / p.gpack);
    p.n_rb = (p.gpack + gqa::fwd_f32_rows_per_tile() - 1) / gqa::fwd_f32_rows_per_tile();
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.num_splits = num_splits;
    p.split_chunk = chunk;
    p.ws_o = ws_o;
    p.ws_lse = ws_lse;
    if (num_splits == 1) return status_from(gqa::launch_fwd_f32(p, d, false, false, false, s));
    hipError_t e = gqa::launch_fwd_f32(p, d, false, false, true, s);
    if (e != hipSuccess) return status_from(e);
    return status_from(
        gqa::launch_decode_combine(ws_o, ws_lse, out, lse, rows, num_splits, d, false, s));
}

int gqa_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, void *out,
                            float *lse, int B, int Hq, int Hkv, int Sk, int d, float scale,
                            int num_splits, int dtype, void *stream) {
    // the same checks as gqa_attn_decode with a workspace of the scratch's
    // size (a stand-in pointer: nothing is launched before they pass)
    const int rc = gqa::validate_decode(q, k_cache, v_cache, out, lse, B, Hq, Hkv, Sk, d, scale,
                                        num_splits, reinterpret_cast<void *>(uintptr_t(256)),
                                        (size_t)GQA_ATTN_NOALLOC_SCRATCH_BYTES, dtype);
    if (rc == GQA_EWORKSPACE) return GQA_ESCRATCH;
    if (rc != GQA_OK) return rc;
    void *ws = nullptr;
    if (num_splits > 1) {
        ws = scratch_address();
        if (!ws) return GQA_ELAUNCH;
    }
    return gqa_attn_decode(q, k_cache, v_cache, out, lse, B, Hq, Hkv, Sk, d, scale, num_splits,
                           ws, num_splits > 1 ? (size_t)GQA_ATTN_NOALLOC_SCRATCH_BYTES : 0, dtype,
                           stream);
}

int gqa_attn_decode_ex(const void *q, const void *k_cache, const void *v_cache, void *out,
                       float *lse, int B, int Hq, int Hkv, int d, float scale,
                       const int32_t *seqlens_k, int max_seqlen_k, const int32_t *block_table,
                       int block_size, int max_blocks_per_seq, int window_left, int kv_dtype,
                       float k_scale, float v_scale, int num_splits, void *workspace,
                       size_t workspace_bytes, void *stream) {
    const int rc = gqa::validate_decode_ex(q, k_cache, v_cache, out, lse, B, Hq, Hkv, d, scale,
                                           seqlens_k, max_seqlen_k, block_table, block_size,
                                           max_blocks_per_seq, window_left, kv_dtype, k_scale,
                                           v_scale, num_splits, workspace, workspace_bytes);
    if (rc != GQA_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *ws_o = nullptr, *ws_lse = nullptr;
    split_workspace(workspace, B, Hq, d, num_splits, ws_o, ws_lse);
    const bool fp8 = kv_dtype == GQA_DTYPE_FP8_E4M3;
    gqa::DecodeParams p{};
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.o = out;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sk = max_seqlen_k;
    p.G = Hq / Hkv;
    p.n_qs = (p.G + 15) / 16;
    p.num_splits = num_splits;
    p.scale_log2 = scale * 1.4426950408889634f * (fp8 ? k_scale : 1.f);
    p.v_scale = fp8 ? v_scale : 1.f;
    p.seqlens = seqlens_k;
    p.block_table = block_table;
    p.log2_block = 0;
    if (block_table)
        while ((1 << p.log2_block) < block_size) ++p.log2_block;
    p.max_blocks = max_blocks_per_seq;
    p.window_left = window_left;
    p.ws_o = ws_o;
    p.ws_lse = ws_lse;
    (void)hipGetLastError();
    hipError_t e = gqa::launch_decode_bf16(p, d, block_table != nullptr, fp8, s);
    if (e != hipSuccess || num_splits == 1) return status_from(e);
    return status_from(gqa::launch_decode_combine(ws_o, ws_lse, out, lse, B * Hq, num_splits, d,
                                                  true, s));
}

}  // extern "C"
