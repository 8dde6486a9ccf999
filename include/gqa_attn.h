/*
 * gqa_attn.h - C ABI of the MI355X (gfx950) fused grouped-query attention
 * forward and split-KV decode.
 *
 * What is computed (per query head h, query row i):
 *   O[i, h, :] = softmax_j(scale * q[i, h, :] . k[j, h / G, :]  (+ causal mask)) . v[j, h / G, :]
 *   LSE[h, i]  = log sum_j exp(scale * q[i, h, :] . k[j, h / G, :])   (natural log)
 * with G = Hq / Hkv query heads sharing each K/V head.
 *
 * Sources (the pages these kernels are built from):
 *  - FlashAttention-2 summary (azimuth.plus): standard attention S = QK^T,
 *    P = row softmax, O = PV; the tiled streaming softmax with a running max
 *    and an unnormalised output rescaled by exp(m_old - m_new), one final
 *    division by l, and the stored statistic L = m + log(l); work split over
 *    batch x heads x query-row blocks; causal masking (diagonal kept) with
 *    whole-tile skipping above the diagonal; GQA through index arithmetic
 *    instead of copying K/V.
 *  - Ultralytics glossary "Grouped Query Attention (GQA)", section "How GQA
 *    works": query head h uses K/V head floor(h / G) (repeat_interleave).
 *  - gitcode GQA batch-size guide, PackGQA paragraph and parameter table:
 *    the query heads of one group packed into one thread block, the
 *    query-head -> K/V-head map fixed ahead of the loop, and the split count
 *    num_splits for the key range.
 *  - Raptor-T abstract (icslab.whu.edu.cn): variable-length inputs without
 *    padding; here packed sequences addressed by prefix offsets.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    calls no allocator; its only state is two static device arrays per GPU,
 *    the variable-length forward's scheduling counters and the scratch of
 *    gqa_attn_decode_noalloc (both described at those entry points). It
 *    never synchronises and never reads device data on the host.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream). Results are ready when the stream has reached the call.
 *  - Tensors are dense and contiguous with head_dim innermost. q, k, v, out
 *    and workspace must be 16-byte aligned; lse and cu_seqlens 4-byte aligned.
 *  - Supported head_dim d: 64 and 128. dtype GQA_DTYPE_BF16 (bf16 in and out,
 *    bf16 matrix-core products with fp32 accumulation) or GQA_DTYPE_FP32
 *    (fp32 in and out, fp32 arithmetic throughout). lse is always fp32.
 *  - `scale` must be finite and > 0 (the usual value is 1/sqrt(d)).
 *  - A row that sees no key (causal with Lq > Lk, or an empty key range) gets
 *    O = 0 and LSE = -inf.
 *  - Every function returns a status; argument errors are reported before
 *    anything is launched. Errors inside device data (e.g. a cu_seqlens array
 *    that is not non-decreasing or exceeds the stated maxima) are not detected
 *    and give undefined results.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_DTYPE_BF16 = 0,
    GQA_DTYPE_FP32 = 1,
    GQA_DTYPE_FP8_E4M3 = 2  /* K/V cache of gqa_attn_decode_ex (OCP e4m3, 1 byte); the inputs
                               of gqa_attn_fwd_fp8 have this format implicitly */
} gqa_dtype;

enum {
    GQA_OK = 0,
    GQA_EINVAL = 1,        /* bad argument: null pointer, bad size, head ratio, scale, alignment */
    GQA_EUNSUPPORTED = 2,  /* head_dim not in {64, 128} or unknown dtype */
    GQA_EWORKSPACE = 3,    /* decode workspace NULL or too small for num_splits > 1 */
    GQA_ELAUNCH = 4,       /* the HIP runtime refused a kernel launch */
    GQA_ESCRATCH = 5       /* gqa_attn_decode_noalloc: partials larger than its static scratch */
};

/* Bytes of the static device scratch behind gqa_attn_decode_noalloc (per GPU). */
#define GQA_ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * gqa_attn_fwd - exact attention forward (prefill / encoder), fixed length or
 * variable length.
 *
 * Fixed length (cu_seqlens_q == cu_seqlens_k == NULL):
 *   q   [B, Sq, Hq,  d]   out [B, Sq, Hq, d] (same dtype as q)
 *   k,v [B, Sk, Hkv, d]   lse [B, Hq, Sq] fp32
 * Variable length (both cu_seqlens given, int32 [B+1] on the device,
 * cu[0] = 0, non-decreasing; sequence b owns query rows cu_q[b]..cu_q[b+1]-1
 * and keys cu_k[b]..cu_k[b+1]-1, no padding):
 *   q   [total_q, Hq,  d]  out [total_q, Hq, d]
 *   k,v [total_k, Hkv, d]  lse [total_q, Hq] fp32 (token-major)
 *   Sq and Sk carry the largest per-sequence query / key length; they size
 *   the launch grid only. A sequence longer than them is undefined.
 * causal != 0 masks key j for query row i when j > i + (Lk - Lq) (per
 * sequence; the diagonal is kept; bottom-right alignment when Lq != Lk).
 * Requirements: B, Hq, Hkv >= 1; Sq, Sk >= 1 for fixed length and >= 0 for
 * variable length; Hq % Hkv == 0; Hkv * d <= 4194304 (one token's K row at
 * most 8 MiB, so per-lane offsets inside a key tile fit 24 bits).
 * Scheduling (bf16 and fp8, variable length): one workgroup per resident
 * slot of the device takes row tiles until none is left, claiming them
 * through nine counters in device memory that the library holds (64 such
 * slots per device, used in turn by successive calls; every call returns its
 * slot to zero). Calls whose executions overlap on one device must not share
 * a slot, so at most 64 variable-length forward calls may be executing on
 * one device at a time. Setting the environment variable
 * GQA_FWD_PERSISTENT=0 before the first call launches one workgroup per row
 * tile instead (as fixed-length calls always do).
 */
int gqa_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                 int dtype, void *stream);

/*
 * gqa_attn_fwd_fp8 - gqa_attn_fwd over fp8 e4m3 inputs (the gitcode GQA
 * batch-size guide's hardware section: FP8 precision to relieve memory
 * bandwidth; its parameter table's precision row). The pages fix no format;
 * the OCP E4M3 byte format is used with one dequantisation scale per tensor:
 * the value of a stored code x is decode(x) * q_scale (resp. k_scale,
 * v_scale).
 *
 * q, k, v: e4m3 codes (1 byte each), in the layouts of gqa_attn_fwd (fixed
 *   or variable length, same cu_seqlens rules); out: bf16 in q's layout;
 *   lse: fp32 as for gqa_attn_fwd.
 * Result: the attention of the dequantised tensors, with the softmax scale
 *   `scale`, computed as follows: scores on the fp8 matrix cores (exact
 *   products of the codes; each sum of 64 of them is formed inside the
 *   matrix core at somewhat less than fp32 precision, measured at about
 *   2^-15 of the score, then accumulated in fp32 and multiplied by scale x
 *   q_scale x k_scale), probabilities rounded to bf16, V widened exactly to
 *   bf16 for the bf16 matrix-core product, O multiplied by v_scale before the
 *   final rounding to bf16.
 * Requirements: those of gqa_attn_fwd; q_scale, k_scale, v_scale finite and
 *   > 0, and scale x q_scale x k_scale finite and > 0. Codes 0x7f / 0xff
 *   (NaN) give undefined results.
 * Errors: GQA_EINVAL, GQA_EUNSUPPORTED (d not in {64, 128}), GQA_ELAUNCH.
 */
int gqa_attn_fwd_fp8(const void *q, const void *k, const void *v, void *out, float *lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, float q_scale,
                     float k_scale, float v_scale, void *stream);

/*
 * gqa_attn_bwd_workspace_bytes - size of the caller-owned workspace of
 * gqa_attn_bwd for B sequences, Hq query heads (of Hkv K/V heads), Sq query
 * and Sk key rows (the largest per-sequence lengths for variable length) and
 * head dim d: two fp32 row statistics per (sequence, head, row) plus padding
 * and, when B x Hkv x ceil(Sk / 128) is below 256 (too few key blocks to
 * fill the chip, so the rows seeing each key block are split into chunks),
 * fp32 partial key and value gradients (2 x 128 x d floats per key block and
 * chunk). Returns 0 for invalid sizes.
 */
size_t gqa_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d);

/*
 * gqa_attn_bwd - gradients of gqa_attn_fwd (FlashAttention-2 summary,
 * backward-pass paragraph: probabilities recomputed from the inputs and the
 * stored LSE; key/value gradients accumulated per key block and summed over
 * the query heads that share each K/V head).
 *
 * Inputs: q, k, v, out and lse exactly as given to / returned by
 * gqa_attn_fwd with the same sizes, causal flag, scale and cu_seqlens, plus
 * dout (the gradient of out, same layout as out). Outputs: dq (layout of q),
 * dk, dv (layout of k, v), overwritten (not accumulated). bf16 only
 * (dtype GQA_DTYPE_BF16; GQA_DTYPE_FP32 gives GQA_EUNSUPPORTED).
 *   dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K, dK = scale dS^T Q, P = exp(scale q k^T - LSE),
 * with dK, dV of K/V head g summed over query heads h with h / G = g.
 * Keys that no query sees get dK = dV = 0; rows that see no key get dQ = 0.
 * workspace: device memory of at least gqa_attn_bwd_workspace_bytes(B, Hq,
 * Hkv, Sq, Sk, d) bytes, 16-byte aligned, contents ignored and overwritten.
 * Errors: as gqa_attn_fwd, plus GQA_EWORKSPACE for a missing or short
 * workspace.
 */
int gqa_attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Sq,
                 int Sk, int d, float scale, int causal, const int32_t *cu_seqlens_q,
                 const int32_t *cu_seqlens_k, void *workspace, size_t workspace_bytes, int dtype,
                 void *stream);

/*
 * gqa_attn_decode_workspace_bytes - size of the caller-owned workspace that
 * gqa_attn_decode / gqa_attn_decode_ex need for num_splits partial results
 * (fp32 normalised partial outputs [num_splits, B*Hq, d], the size rounded up
 * to 256 bytes, followed by fp32 partial LSEs [num_splits, B*Hq]); the
 * contents need no initialisation and are overwritten by every call.
 * Returns 0 when num_splits == 1 (no workspace needed) and 0 for invalid
 * sizes (num_splits < 1, B, Hq < 1, d not in {64, 128}).
 */
size_t gqa_attn_decode_workspace_bytes(int B, int Hq, int d, int num_splits);

/*
 * gqa_attn_decode - one new query token per sequence attending, without a
 * mask, to its whole K/V cache, with the key range cut into num_splits
 * contiguous ranges (gitcode GQA guide's num_splits) whose partial results are
 * merged through their log-sum-exps:
 *   L = M + log sum_s exp(L_s - M), M = max_s L_s;  O = sum_s exp(L_s - L) O_s.
 *   q [B, Hq, d]; k_cache, v_cache [B, Sk, Hkv, d]; out [B, Hq, d]; lse [B, Hq].
 * Split s covers keys [s*c, min(Sk, (s+1)*c)) with c = ceil(Sk/num_splits)
 * rounded up to a multiple of 64; trailing splits may be empty and then
 * contribute nothing. 1 <= num_splits <= 64. For num_splits > 1 the caller
 * passes a device workspace of at least gqa_attn_decode_workspace_bytes().
 * Results agree for every num_splits up to rounding.
 */
int gqa_attn_decode(const void *q, const void *k_cache, const void *v_cache, void *out,
                    float *lse, int B, int Hq, int Hkv, int Sk, int d, float scale,
                    int num_splits, void *workspace, size_t workspace_bytes,
                    int dtype, void *stream);

/*
 * gqa_attn_decode_noalloc - gqa_attn_decode without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. It allocates nothing
 * (no hipMalloc, hipFree or allocating library call); the caller passes the
 * inputs and outputs exactly as for gqa_attn_decode, and for num_splits > 1
 * the fp32 split partials go to a static device array of
 * GQA_ATTN_NOALLOC_SCRATCH_BYTES bytes (16 MiB) that the library holds on
 * every GPU it runs on until the process ends (its address is looked up once
 * per device, on the first call with that device current). Nothing in it must
 * start at zero: every split writes its LSE (-inf when empty) and the merge
 * reads a split's O only when its LSE is finite.
 * Limit: gqa_attn_decode_workspace_bytes(B, Hq, d, num_splits) must not exceed
 * GQA_ATTN_NOALLOC_SCRATCH_BYTES (B * Hq * (d + 1) * 4 * num_splits bytes,
 * rounded; e.g. B 64, Hq 32, d 128, num_splits 8 needs 8.5 MB), else
 * GQA_ESCRATCH before anything is launched. num_splits == 1 uses no scratch.
 * All calls on one GPU share its scratch, which keeps the last call's
 * contents: calls that overlap on one GPU (different streams, or different
 * host threads without ordering) race; issue them on one stream.
 * Errors: as gqa_attn_decode (GQA_EWORKSPACE cannot occur), GQA_ESCRATCH, and
 * GQA_ELAUNCH also when the scratch address cannot be obtained.
 */
int gqa_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, void *out,
                            float *lse, int B, int Hq, int Hkv, int Sk, int d, float scale,
                            int num_splits, int dtype, void *stream);

/*
 * gqa_attn_decode_ex - decode over a ragged, optionally paged, optionally
 * windowed, bf16 or fp8 K/V cache (the same split-KV method and LSE merge as
 * gqa_attn_decode).
 *
 * Queries: q [B, Hq, d] bf16 -> out [B, Hq, d] bf16, lse [B, Hq] fp32.
 * Cache, contiguous (block_table == NULL): k_cache, v_cache [B, max_seqlen_k, Hkv, d].
 * Cache, paged (block_table != NULL, the fixed-size KV blocks named in the
 *   Ultralytics glossary's PagedAttention item): k_cache, v_cache
 *   [num_blocks, block_size, Hkv, d]; block_table int32 [B, max_blocks_per_seq]
 *   on the device; key j of sequence b is slot j % block_size of block
 *   block_table[b][j / block_size]. block_size must be a power of two
 *   (1 .. 4096) and max_blocks_per_seq >= ceil(max_seqlen_k / block_size).
 * seqlens_k: int32 [B] on the device (keys held by each sequence, 0 ..
 *   max_seqlen_k; values outside that range are clamped into it), or NULL
 *   when every sequence holds max_seqlen_k keys.
 * window_left: -1 attends to every cached key; W >= 0 restricts each query to
 *   the last W + 1 keys of its sequence (keys j >= L - 1 - W), the sliding
 *   window of the glossary's related-techniques list.
 * kv_dtype: GQA_DTYPE_BF16, or GQA_DTYPE_FP8_E4M3 with per-tensor
 *   dequantisation scales (stored value x k_scale / v_scale; both ignored for
 *   bf16). fp8 values are widened exactly to bf16 for the matrix cores.
 * Splits: the visible keys of each sequence are cut into num_splits
 *   contiguous ranges of ceil(n / num_splits) keys rounded up to a multiple
 *   of 64 (trailing ranges may be empty); workspace as for gqa_attn_decode.
 *   With seqlens_k and B <= 256 the workgroups take the sequences longest
 *   first. A sequence with no visible key gets O = 0 and LSE = -inf.
 * Errors: GQA_EINVAL for bad sizes, pointers, alignment, scales, block
 * geometry or window; GQA_EUNSUPPORTED for d not in {64, 128} or an
 * unsupported kv_dtype; GQA_EWORKSPACE as for gqa_attn_decode.
 */
int gqa_attn_decode_ex(const void *q, const void *k_cache, const void *v_cache, void *out,
                       float *lse, int B, int Hq, int Hkv, int d, float scale,
                       const int32_t *seqlens_k, int max_seqlen_k, const int32_t *block_table,
                       int block_size, int max_blocks_per_seq, int window_left, int kv_dtype,
                       float k_scale, float v_scale, int num_splits, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * gqa_attn_decode_num_splits - a split count for gqa_attn_decode /
 * gqa_attn_decode_ex on MI355X (the gitcode GQA guide's num_splits knob; its
 * A100/H100 table is prior art for other chips and is not used).
 *
 * Measured rule: a decode launch has B * Hkv * ceil(G / 16) workgroups per
 * split; splits are added until there are about 192 or more of them
 * (units >= 192 -> 1, >= 96 -> 2, >= 48 -> 4, >= 12 -> 8, else 16). A ragged
 * batch (ragged != 0: per-sequence lengths that differ) takes at least 2, so
 * that its longest sequences are cut and scheduled first, unless a sliding
 * window of at most half of max_seqlen_k evens the visible ranges out (most
 * sequences then see exactly window_left + 1 keys). The count is then
 * halved while a split would get fewer than 512 keys of the longest visible
 * range (max_seqlen_k, or window_left + 1 when smaller). On a split-count
 * sweep of contiguous bf16 caches with 32 query and 8 K/V heads (B 1..128,
 * 512..32768 keys, d 64 and 128; 64 points) the pick is the fastest count at
 * 40 points, its time is the best count's at the median and at most 1.29
 * times it; the largest losses are on short calls (8-20 us: B <= 4 at 2048
 * keys), where 8 or 16 splits beat the picked 4, and on long caches at
 * large B at d 64, where 16 splits run 15-17 % faster than the 1 picked.
 * Returns 0 for invalid arguments (same rules as gqa_attn_decode_ex).
 */
int gqa_attn_decode_num_splits(int B, int Hq, int Hkv, int d, int max_seqlen_k, int window_left,
                               int ragged);

/* gqa_attn_strerror - static, NUL-terminated description of a status code. */
const char *gqa_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
