// Fused attention prefill with fp32 inputs: fp32 products, fp32 accumulation,
// fp32 output.  Same problem and masks as the bf16 kernel; this variant keeps
// full fp32 precision (no 16-bit rounding of Q, K or P anywhere), which the
// fp32 tolerance of the method needs.
//
// One workgroup = 8 wavefronts = 16 query rows of one (batch, head).  Four
// consecutive lanes share a query row, each holding a quarter of its dims
// (16-byte chunks c = sub, sub + 4, ...), so a score is four partial dot
// products summed across the quad.  The wavefronts split the row block's
// visible key tiles (16 keys each; wavefront w takes tiles w, w + 8, ...;
// two wavefronts per SIMD hide each other's LDS and memory latency),
// each keeping its own running max and sum per row (hwcomputing.csdn.net
// page, section 2.2), and merge their partial results through LDS once at
// the end: the serial work of a lane is a thirty-second of one lane per row over
// all keys.  Each wavefront stages its tiles in LDS private to it, so the
// tile loop needs no workgroup barrier.  Tiles outside the causal / window /
// valid-length band are skipped and padding rows are zero-filled, never
// read (jsqmd.com page, section 二 "causal mask and decode"; agent.csdn.net
// BERT page, chapter 四).
#include "fa_internal.h"

#include <cmath>

namespace fa {
namespace {

constexpr int BM = kPrefillF32BM;   // query rows per workgroup
constexpr int NW = 8;               // wavefronts per workgroup
constexpr int BN = 16;              // keys per tile
constexpr float LN2 = 0.693147180559945309f;

// Sum over the 4 lanes of a quad; every lane gets the total.
__device__ __forceinline__ float quad_sum(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    return x;
}

template <int D>
__global__ __launch_bounds__(NW * 64) void prefill_f32_kernel(PrefillArgs a) {
    static_assert(BM * 4 == 64, "one wavefront of lanes covers the row block");
    constexpr int CH = D / 4;                   // 16-byte chunks per row
    constexpr int CPL = CH / 4;                 // chunks per lane
    __shared__ __attribute__((aligned(16))) float Ks[NW][BN][D];
    __shared__ __attribute__((aligned(16))) float Vs[NW][BN][D];
    __shared__ float mml[NW][BM][2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rl = lane >> 2, sub = lane & 3;   // row of the block, quarter of the dims
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

    // key tiles the row block can see: [t_begin, t_end)
    int kv_lo = 0, kv_hi = Lk;
    if (r0 < Lq) {
        const int q_last = min(q0 + BM, Lq) - 1;
        if (a.causal) kv_hi = min(kv_hi, q_last + offset + 1);
        if (W > 0) kv_lo = max(0, r0 + offset - W + 1);
    }
    const int t_begin = kv_lo / BN;
    int t_end = (kv_hi + BN - 1) / BN;
    if (r0 >= min(q0 + BM, Lq) || kv_hi <= kv_lo) t_end = t_begin;

    const float *Qp = (const float *)a.q + b * a.q_sb + h * a.q_sh;
    const float *Kp = (const float *)a.k + b * a.k_sb + kvh * a.k_sh;
    const float *Vp = (const float *)a.v + b * a.v_sb + kvh * a.v_sh;

    // RoPE: pair (2p, 2p + 1) at position m turns by the table's angle
    // (x, y) -> (x c - y s, x s + y c); queries sit at i + Lk - Lq, keys at j.
    // A 16-byte chunk c holds pairs 2c and 2c + 1.
    const int rhalf = a.rotary_dim / 2;
    auto rotate4 = [&](float4 x, int m, int c) __attribute__((always_inline)) -> float4 {
        if (4 * c >= a.rotary_dim) return x;
        const float *cr = a.rope_cos + (int64_t)m * rhalf + 2 * c;
        const float *sr = a.rope_sin + (int64_t)m * rhalf + 2 * c;
        const float c0 = cr[0], c1 = cr[1], s0 = sr[0], s1 = sr[1];
        return make_float4(__builtin_fmaf(x.x, c0, -x.y * s0), __builtin_fmaf(x.x, s0, x.y * c0),
                           __builtin_fmaf(x.z, c1, -x.w * s1), __builtin_fmaf(x.z, s1, x.w * c1));
    };

    // this lane's quarter of its query row (zero outside the valid rows)
    const int qi = q0 + rl;
    const int pos = qi + offset;
    const bool row_live = qi < Lq && qi >= q_first;
    float4 q[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
        const int c = sub + 4 * u;
        q[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_live) {
            q[u] = rotate4(*(const float4 *)(Qp + (int64_t)qi * a.q_ss + 4 * c), pos, c);
        }
    }

    float4 o[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = a.scale_log2;
    // ALiBi in raw score units: scale * s + bias = scale * (s + bias / scale)
    const float alibi_raw = a.alibi ? -a.alibi[h] / a.scale : 0.f;
    // explicit additive mask row of this lane's query (clamped into the
    // tensor for rows of a partial block), in raw score units
    const float *mrow = a.mask ? (const float *)a.mask + b * a.m_sb + h * a.m_sh +
                                     (int64_t)min(qi, a.seqlen_q - 1) * a.m_ss
                               : nullptr;
    const float inv_scale = 1.f / a.scale;

    for (int t = t_begin + wave; t < t_end; t += NW) {
        const int k0 = t * BN;
        // stage this wavefront's tile: BN rows x CH chunks of K and of V
#pragma unroll
        for (int i = 0; i < BN * CH / 64; ++i) {
            const int n = 64 * i + lane;
            const int r = n / CH, c = n - (n / CH) * CH;
            const int j = k0 + r;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (j < Lk) {
                kx = rotate4(*(const float4 *)(Kp + (int64_t)j * a.k_ss + 4 * c), j, c);
                vx = *(const float4 *)(Vp + (int64_t)j * a.v_ss + 4 * c);
            }
            *(float4 *)&Ks[wave][r][4 * c] = kx;
            *(float4 *)&Vs[wave][r][4 * c] = vx;
        }
        // this wavefront's LDS writes land before any of its lanes reads them
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();

        float s[BN];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < BN; ++jj) {
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                const float4 kx = *(const float4 *)&Ks[wave][jj][4 * (sub + 4 * u)];
                acc = __builtin_fmaf(q[u].x, kx.x, acc);
                acc = __builtin_fmaf(q[u].y, kx.y, acc);
                acc = __builtin_fmaf(q[u].z, kx.z, acc);
                acc = __builtin_fmaf(q[u].w, kx.w, acc);
            }
            acc = quad_sum(acc);
            const int key = k0 + jj;
            bool vis = key < Lk && row_live;
            if (a.causal) vis = vis && key <= pos;
            if (W > 0) vis = vis && key > pos - W;
            if (a.alibi) acc = __builtin_fmaf(fabsf((float)(pos - key)), alibi_raw, acc);
            if (mrow && key < a.seqlen_k) acc = __builtin_fmaf(mrow[key], inv_scale, acc);
            s[jj] = vis ? acc : -INFINITY;
            mx = fmaxf(mx, s[jj]);
        }
        const float m_new = fmaxf(m_run, mx * c2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int jj = 0; jj < BN; ++jj) {
            s[jj] = exp2f(__builtin_fmaf(s[jj], c2, -m_use));
            psum += s[jj];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            float4 acc = make_float4(o[u].x * alpha, o[u].y * alpha, o[u].z * alpha, o[u].w * alpha);
#pragma unroll
            for (int jj = 0; jj < BN; ++jj) {
                const float4 vx = *(const float4 *)&Vs[wave][jj][4 * (sub + 4 * u)];
                acc.x = __builtin_fmaf(s[jj], vx.x, acc.x);
                acc.y = __builtin_fmaf(s[jj], vx.y, acc.y);
                acc.z = __builtin_fmaf(s[jj], vx.z, acc.z);
                acc.w = __builtin_fmaf(s[jj], vx.w, acc.w);
            }
            o[u] = acc;
        }
        // every lane's reads of the tile are done before the next one is staged
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
    }

    // ---- merge the wavefronts, normalise once, write O and LSE ------------
    __syncthreads();                              // every wavefront is done with its tiles
    float *mo = &Ks[0][0][0];                     // [NW][BM][D] partial P.V rows
    static_assert(BM <= BN, "the merge fits the K buffers");
#pragma unroll
    for (int u = 0; u < CPL; ++u) *(float4 *)&mo[(wave * BM + rl) * D + 4 * (sub + 4 * u)] = o[u];
    if (sub == 0) {
        mml[wave][rl][0] = m_run;
        mml[wave][rl][1] = l_run;
    }
    __syncthreads();
    if (wave == 0 && qi < a.seqlen_q) {
        float M = mml[0][rl][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, mml[w][rl][0]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float wt[NW], L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            wt[w] = exp2f(mml[w][rl][0] - M_use);
            L = __builtin_fmaf(wt[w], mml[w][rl][1], L);
        }
        const bool row_ok = qi < Lq && L > 0.f;
        const float inv = row_ok ? 1.f / L : 0.f;
        float *orow = (float *)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_ss;
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const int c = sub + 4 * u;
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float4 x = *(const float4 *)&mo[(w * BM + rl) * D + 4 * c];
                acc.x = __builtin_fmaf(wt[w], x.x, acc.x);
                acc.y = __builtin_fmaf(wt[w], x.y, acc.y);
                acc.z = __builtin_fmaf(wt[w], x.z, acc.z);
                acc.w = __builtin_fmaf(wt[w], x.w, acc.w);
            }
            *(float4 *)(orow + 4 * c) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        }
        if (a.lse && sub == 0) {
            float *lrow = a.lse + ((int64_t)b * a.heads_q + h) * a.seqlen_q;
            lrow[qi] = row_ok ? (M_use + log2f(L)) * LN2 : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)a.num_q_tiles * a.heads_q * a.batch);
    const dim3 block(NW * 64);
    if (head_dim == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace fa
