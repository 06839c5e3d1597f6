// Fused attention prefill with fp32 inputs: fp32 products, fp32 accumulation,
// fp32 output.  Same problem and masks as the bf16 kernel; this variant keeps
// full fp32 precision (no 16-bit rounding of Q, K or P anywhere), which the
// fp32 tolerance of the method needs.
//
// One workgroup = one wavefront = 64 query rows of one (batch, head); each
// lane owns one query row.  K/V tiles of 32 keys are staged in LDS and read
// by all lanes as broadcasts; the row keeps a running max and running sum
// (hwcomputing.csdn.net page, section 2.2) and is normalised once at the end.
// Tiles outside the causal / window / valid-length band are skipped and
// padding rows are zero-filled, never read (jsqmd.com page, section 二
// "causal mask and decode"; agent.csdn.net BERT page, chapter 四).
#include "fa_internal.h"

#include <cmath>

namespace fa {
namespace {

constexpr int BM = kPrefillF32BM;   // query rows per workgroup (= lanes)
constexpr int BN = 32;              // keys per tile
constexpr float LN2 = 0.693147180559945309f;

template <int D>
__global__ __launch_bounds__(BM) void prefill_f32_kernel(PrefillArgs a) {
    __shared__ float Qs[BM][D + 1];
    __shared__ __attribute__((aligned(16))) float Ks[BN][D];
    __shared__ __attribute__((aligned(16))) float Vs[BN][D];

    const int tid = threadIdx.x;
    const int bh_count = a.batch * a.heads_q;
    const int rank = blockIdx.x / bh_count;
    const int bh = blockIdx.x - rank * bh_count;
    const int b = bh / a.heads_q;
    const int h = bh - b * a.heads_q;
    const int qtile = a.causal ? (a.num_q_tiles - 1 - rank) : rank;
    const int kvh = h / a.group;

    int Lq = a.seqlen_q, Lk = a.seqlen_k;
    if (a.seqlens_q) Lq = min(max(a.seqlens_q[b], 0), a.seqlen_q);
    if (a.seqlens_k) Lk = min(max(a.seqlens_k[b], 0), a.seqlen_k);
    const int q0 = qtile * BM;
    const int offset = Lk - Lq;
    const int W = a.window_left;
    // RoPE: rows before position 0 (i < Lq - Lk) have no angle in the tables
    // and see no key; the valid rows are [q_first, Lq)
    const int q_first = a.rotary_dim > 0 ? max(0, -offset) : 0;
    const int r0 = max(q0, q_first);

    int kv_lo = 0, kv_hi = Lk;
    if (r0 < Lq) {
        const int q_last = min(q0 + BM, Lq) - 1;
        if (a.causal) kv_hi = min(kv_hi, q_last + offset + 1);
        if (W > 0) kv_lo = max(0, r0 + offset - W + 1);
    }
    int t_begin = kv_lo / BN;
    int t_end = (kv_hi + BN - 1) / BN;
    if (r0 >= min(q0 + BM, Lq) || kv_hi <= kv_lo) t_end = t_begin;

    const float *Qp = (const float *)a.q + b * a.q_sb + h * a.q_sh;
    const float *Kp = (const float *)a.k + b * a.k_sb + kvh * a.k_sh;
    const float *Vp = (const float *)a.v + b * a.v_sb + kvh * a.v_sh;

    // RoPE: pair (2p, 2p + 1) at position m turns by the table's angle
    // (x, y) -> (x c - y s, x s + y c); queries sit at i + Lk - Lq, keys at j
    const int rhalf = a.rotary_dim / 2;
    auto rotate = [&](float &x, float &y, int m, int p) {
        if (p < rhalf) {
            const float c = a.rope_cos[(int64_t)m * rhalf + p], sn = a.rope_sin[(int64_t)m * rhalf + p];
            const float x0 = x;
            x = __builtin_fmaf(x0, c, -y * sn);
            y = __builtin_fmaf(x0, sn, y * c);
        }
    };

    // stage this workgroup's query rows (zero outside the valid length), a
    // pair of dims per step
    for (int idx = tid; idx < BM * (D / 2); idx += BM) {
        const int r = idx / (D / 2), p = idx - (idx / (D / 2)) * (D / 2);
        const int i = q0 + r;
        float x = 0.f, y = 0.f;
        if (i < Lq && i >= q_first) {
            x = Qp[(int64_t)i * a.q_ss + 2 * p];
            y = Qp[(int64_t)i * a.q_ss + 2 * p + 1];
            rotate(x, y, i + offset, p);
        }
        Qs[r][2 * p] = x;
        Qs[r][2 * p + 1] = y;
    }

    const int qi = q0 + tid;
    const int pos = qi + offset;
    float o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;
    // ALiBi in raw score units: scale * s + bias = scale * (s + bias / scale)
    const float alibi_raw = a.alibi ? -a.alibi[h] / a.scale : 0.f;
    // explicit additive mask row of this lane's query (clamped into the
    // tensor for rows of a partial tile), in raw score units
    const float *mrow = a.mask ? (const float *)a.mask + b * a.m_sb + h * a.m_sh +
                                     (int64_t)min(qi, a.seqlen_q - 1) * a.m_ss
                               : nullptr;
    const float inv_scale = 1.f / a.scale;

    for (int t = t_begin; t < t_end; ++t) {
        const int k0 = t * BN;
        __syncthreads();
        for (int idx = tid; idx < BN * (D / 2); idx += BM) {
            const int r = idx / (D / 2), p = idx - (idx / (D / 2)) * (D / 2);
            const int j = k0 + r;
            float x = 0.f, y = 0.f;
            if (j < Lk) {
                x = Kp[(int64_t)j * a.k_ss + 2 * p];
                y = Kp[(int64_t)j * a.k_ss + 2 * p + 1];
                rotate(x, y, j, p);
            }
            Ks[r][2 * p] = x;
            Ks[r][2 * p + 1] = y;
        }
        for (int idx = tid; idx < BN * D; idx += BM) {
            const int r = idx / D, d = idx - (idx / D) * D;
            const int j = k0 + r;
            Vs[r][d] = (j < Lk) ? Vp[(int64_t)j * a.v_ss + d] : 0.f;
        }
        __syncthreads();

        float s[BN];
#pragma unroll
        for (int j = 0; j < BN; ++j) s[j] = 0.f;
        for (int d = 0; d < D; ++d) {
            const float qd = Qs[tid][d];
#pragma unroll
            for (int j = 0; j < BN; ++j) s[j] = __builtin_fmaf(qd, Ks[j][d], s[j]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            const int key = k0 + j;
            bool vis = key < Lk && qi >= q_first;
            if (a.causal) vis = vis && key <= pos;
            if (W > 0) vis = vis && key > pos - W;
            if (a.alibi) s[j] = __builtin_fmaf(fabsf((float)(pos - key)), alibi_raw, s[j]);
            if (mrow && key < a.seqlen_k) s[j] = __builtin_fmaf(mrow[key], inv_scale, s[j]);
            s[j] = vis ? s[j] : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx * c2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            s[j] = exp2f(__builtin_fmaf(s[j], c2, -m_use));
            psum += s[j];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float acc = o[d] * alpha;
#pragma unroll
            for (int j = 0; j < BN; ++j) acc = __builtin_fmaf(s[j], Vs[j][d], acc);
            o[d] = acc;
        }
    }

    if (qi < a.seqlen_q) {
        const bool row_ok = qi < Lq && l_run > 0.f;
        const float inv = row_ok ? 1.f / l_run : 0.f;
        float *orow = (float *)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_ss;
#pragma unroll
        for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
        if (a.lse) {
            float *lrow = a.lse + ((int64_t)b * a.heads_q + h) * a.seqlen_q;
            lrow[qi] = row_ok ? (m_run + log2f(l_run)) * LN2 : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)a.num_q_tiles * a.heads_q * a.batch);
    const dim3 block(BM);
    if (head_dim == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace fa
