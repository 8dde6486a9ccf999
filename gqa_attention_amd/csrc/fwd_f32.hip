// Fused GQA attention forward in fp32 (fp32 in, fp32 arithmetic, fp32 out).
//
// The same tiled streaming softmax as the bf16 kernel (FlashAttention-2
// summary, deferred-normalisation equation and the L = m + log(l) statistic),
// computed on the vector ALUs in fp32 so that the result stays within 1e-5 of
// the exact value. It also serves split-KV decode in fp32: with `SPLIT`, a
// workgroup covers one contiguous key range (gitcode GQA guide, num_splits)
// and writes that range's normalised output and log-sum-exp as partials.
//
// Layout: a workgroup owns 32 packed query rows (rho = position * gpack +
// head_in_group, as in the bf16 kernel) and 8 lanes per row; lane `sub` of a
// row holds head_dim elements sub, sub + 8, ... so the 8 lanes of a row read
// 8 consecutive floats of a K/V row from LDS. Dot products are reduced over
// the 8 lanes with xor shuffles. K/V tiles of 32 keys are staged in LDS.

#include "device_util.h"
#include "params.h"

namespace gqa {

namespace {

constexpr int ROWS = 32;   // packed query rows per workgroup
constexpr int TKEYS = 32;  // keys per tile
constexpr int NTHREADS = 256;

template <int D, bool CAUSAL, bool VARLEN, bool SPLIT>
__global__ __launch_bounds__(NTHREADS) void fwd_f32_kernel(FwdParams p) {
    constexpr int DL = D / 8;  // elements per lane
    __shared__ __attribute__((aligned(16))) float Kf[TKEYS * D];
    __shared__ __attribute__((aligned(16))) float Vf[TKEYS * D];

    const int tid = threadIdx.x;
    const int rloc = tid >> 3, sub = tid & 7;

    const int pid = blockIdx.x;
    const int hg = pid % p.n_hg;
    const int rest = pid / p.n_hg;
    const int rb = rest % p.n_rb;
    const int split = rest / p.n_rb;
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
    const int row0 = rb * ROWS;
    if (row0 >= rows_total) return;

    int k_lo = 0, k_hi = Lk;
    if (SPLIT) {
        k_lo = min(Lk, split * p.split_chunk);
        k_hi = min(Lk, k_lo + p.split_chunk);
    }
    const int shift = Lk - Lq;
    int kend = k_hi;
    if (CAUSAL) {
        const int last = min(row0 + ROWS, rows_total) - 1;
        kend = min(k_hi, last / p.gpack + 1 + shift);
    }

    const int rho = row0 + rloc;
    const bool row_ok = rho < rows_total;
    const int pos = rho / p.gpack;
    const int head = qh0 + (rho - pos * p.gpack);
    const int row_kend = CAUSAL ? min(k_hi, pos + 1 + shift) : k_hi;

    float qv[DL], o[DL];
    {
        const float *qrow = (const float *)p.q + ((int64_t)(q_tok0 + pos) * p.Hq + head) * D;
#pragma unroll
        for (int i = 0; i < DL; ++i) {
            qv[i] = row_ok ? qrow[sub + 8 * i] : 0.f;
            o[i] = 0.f;
        }
    }
    float m_run = -INFINITY, l_run = 0.f;

    const int64_t kv_stride = (int64_t)p.Hkv * D;
    const float *kbase = (const float *)p.k + ((int64_t)k_tok0 * p.Hkv + kvh) * D;
    const float *vbase = (const float *)p.v + ((int64_t)k_tok0 * p.Hkv + kvh) * D;

    for (int t0 = k_lo; t0 < kend; t0 += TKEYS) {
        // stage K, V rows [t0, t0 + TKEYS) (zeros past kend)
        for (int c = tid; c < TKEYS * D / 4; c += NTHREADS) {
            const int r = c / (D / 4), c4 = c % (D / 4);
            const int key = t0 + r;
            float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
            if (key < kend) {
                kv4 = *(const float4 *)(kbase + key * kv_stride + c4 * 4);
                vv4 = *(const float4 *)(vbase + key * kv_stride + c4 * 4);
            }
            *(float4 *)(&Kf[r * D + c4 * 4]) = kv4;
            *(float4 *)(&Vf[r * D + c4 * 4]) = vv4;
        }
        __syncthreads();

        float s[TKEYS];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < TKEYS; ++j) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < DL; ++i) part = fmaf(qv[i], Kf[j * D + sub + 8 * i], part);
            part += __shfl_xor(part, 1, 8);
            part += __shfl_xor(part, 2, 8);
            part += __shfl_xor(part, 4, 8);
            const float sc = (t0 + j < row_kend) ? part * p.scale : -INFINITY;
            s[j] = sc;
            tmax = fmaxf(tmax, sc);
        }
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = expf(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DL; ++i) o[i] *= alpha;
#pragma unroll
        for (int j = 0; j < TKEYS; ++j) {
            const float pj = expf(s[j] - m_use);
            l_run += pj;
#pragma unroll
            for (int i = 0; i < DL; ++i) o[i] = fmaf(pj, Vf[j * D + sub + 8 * i], o[i]);
        }
        __syncthreads();
    }

    if (!row_ok) return;
    const bool empty = !(l_run > 0.f);
    const float inv = empty ? 0.f : 1.f / l_run;
    const float lse = empty ? -INFINITY : m_run + logf(l_run);
    if (SPLIT) {
        // decode partials: one query position, partial row = b * Hq + head
        const int64_t prow = (int64_t)split * p.B * p.Hq + (int64_t)b * p.Hq + head;
#pragma unroll
        for (int i = 0; i < DL; ++i) p.ws_o[prow * D + sub + 8 * i] = o[i] * inv;
        if (sub == 0) p.ws_lse[prow] = lse;
    } else {
        float *orow = (float *)p.o + ((int64_t)(q_tok0 + pos) * p.Hq + head) * D;
#pragma unroll
        for (int i = 0; i < DL; ++i) orow[sub + 8 * i] = o[i] * inv;
        if (sub == 0) {
            const int64_t li = VARLEN ? (int64_t)(q_tok0 + pos) * p.Hq + head
                                      : ((int64_t)b * p.Hq + head) * p.Sq + pos;
            p.lse[li] = lse;
        }
    }
}

template <int D, bool CAUSAL, bool VARLEN, bool SPLIT>
hipError_t launch_t(const FwdParams &p, hipStream_t s) {
    const long long grid = (long long)p.n_hg * p.n_rb * (SPLIT ? p.num_splits : 1);
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, VARLEN, SPLIT>), dim3((unsigned)grid),
                       dim3(NTHREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int fwd_f32_rows_per_tile() { return ROWS; }

hipError_t launch_fwd_f32(const FwdParams &p, int d, bool causal, bool varlen, bool split,
                          hipStream_t s) {
    if (split) {
        if (varlen || causal) return hipErrorInvalidValue;
        if (d == 64) return launch_t<64, false, false, true>(p, s);
        if (d == 128) return launch_t<128, false, false, true>(p, s);
        return hipErrorInvalidValue;
    }
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

}  // namespace gqa
