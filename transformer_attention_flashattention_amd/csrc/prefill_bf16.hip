// Fused attention prefill, bf16 inputs, bf16 MFMA with fp32 accumulation,
// for gfx950 (CDNA4).
//
// What is computed (per query row i of head h, batch b):
//   O_i = sum_j softmax_j(scale * q_i . k_j) v_j over visible keys j,
//   LSE_i = ln sum_j exp(scale * q_i . k_j)
// with the score matrix never leaving the chip: query rows are split into
// row blocks, keys/values into column blocks, and each row block walks the
// column blocks it can see, keeping a running row max and running row sum
// (ops-transformer practice page, jsqmd.com, section 二 "fused computation
// idea": Q split by rows, K/V by columns, reduction done on chip;
// hwcomputing.csdn.net page, section 2.2: max subtraction for a stable
// exp, block-local maxima corrected to one common maximum, fp32 for max,
// exp and normalisation while the matrix products run in 16-bit).
//
// Work decomposition (one workgroup = 4 wavefronts = 128 query rows):
//   * grid = query tiles x heads x batch; heads and batches are independent
//     work items spread over all CUs (jsqmd.com page, section 二 "multi-head
//     parallel strategy").  Consecutive workgroup ids differ in (batch, head)
//     first, so the dispatcher's round-robin over the 8 XCDs keeps each head's
//     K/V inside one XCD's L2; under a causal mask the longest query tiles are
//     dispatched first.
//   * each KV tile of 64 keys is staged in LDS (double buffered: the next tile
//     is fetched from HBM into registers while the current one is computed,
//     then written to the other LDS buffer -- the two-region ping-pong of the
//     hwcomputing.csdn.net page, section 2.1).
//   * the causal / window / valid-length masks are index arithmetic: tiles
//     wholly outside the visible band are never visited, and the element mask
//     runs only on tiles that cross a boundary (jsqmd.com page, section 二
//     "causal mask and decode").  Keys at or beyond the valid length are
//     zero-filled, never read (agent.csdn.net BERT page, chapter 四).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, 64 lanes):
//   S^T[key][query] = K Q^T : A = K rows from LDS, B = Q held in registers.
//     The accumulator gives each lane one query column and 16 of its 32
//     keys, so row max / row sum are lane-local except for one exchange with
//     the partner lane (lane ^ 32) holding the other 16 keys.
//   O^T[dim][query] += V^T P^T : A = V^T from LDS, B = P^T straight from the
//     S^T accumulator registers converted to bf16.  The contraction order of
//     an MFMA is free as long as A and B agree, so K rows are fetched in a
//     permuted order (bits 2 and 3 of the row index swapped) that makes each
//     lane's 8 consecutive accumulator registers cover 8 consecutive keys --
//     exactly one 16-byte row piece of V^T.
//   V^T is written to LDS transposed (4 keys x 8 dims per thread, repacked in
//   registers) with an XOR swizzle of its 16-byte chunks so that both the
//   transposing writes and the MFMA operand reads are free of bank conflicts
//   to within 2-way.
#include "fa_internal.h"

#include <cmath>

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr int BM = kPrefillBM;   // query rows per workgroup
constexpr int BN = 64;           // keys per KV tile
constexpr int NTHREADS = 256;
constexpr float LN2 = 0.693147180559945309f;

// Row permutation of a 32-key sub-block: swap bits 2 and 3.
__device__ __forceinline__ int perm32(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// XOR swizzle of the 16-byte chunk index within a V^T row of 64 keys.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, r);
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2)))
void prefill_bf16_kernel(PrefillArgs a) {
    constexpr int KSTEPS = D / 16;        // MFMA k-steps over head_dim for S
    constexpr int DBLK = D / 32;          // 32-dim row blocks of O^T
    constexpr int KS = D + 8;             // K row stride in LDS (elements)
    constexpr int K_ELEMS = BN * KS;
    constexpr int STAGE = K_ELEMS + D * BN;
    constexpr int DCH = D / 8;            // 16-byte chunks per head_dim row
    constexpr int KLOADS = BN * DCH / NTHREADS;
    constexpr int VUNITS = (BN / 4) * DCH;   // (4-key group, dim chunk) units

    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // ---- work item --------------------------------------------------------
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
    const int offset = Lk - Lq;           // bottom-right causal alignment
    const int W = a.window_left;

    int kv_lo = 0, kv_hi = Lk;
    if (q0 < Lq) {
        const int q_last = min(q0 + BM, Lq) - 1;
        if (a.causal) kv_hi = min(kv_hi, q_last + offset + 1);
        if (W > 0) kv_lo = max(0, q0 + offset - W + 1);
    }
    int t_begin = kv_lo / BN;
    int t_end = (kv_hi + BN - 1) / BN;
    if (q0 >= Lq || kv_hi <= kv_lo) t_end = t_begin;   // nothing visible

    const unsigned short *Qp = (const unsigned short *)a.q + b * a.q_sb + h * a.q_sh;
    const unsigned short *Kp = (const unsigned short *)a.k + b * a.k_sb + kvh * a.k_sh;
    const unsigned short *Vp = (const unsigned short *)a.v + b * a.v_sb + kvh * a.v_sh;

    const int q0w = q0 + wave * 32;       // first query row of this wave
    const int qi = q0w + l32;             // this lane's query row

    // ---- Q fragment (B operand), zero for rows outside the valid length ---
    bf16x8 qf[KSTEPS];
    {
        const bool ok = qi < Lq;
        const unsigned short *row = Qp + (int64_t)qi * a.q_ss + half * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok) v = *(const u32x4 *)(row + ks * 16);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- global -> register -> LDS staging of one KV tile ------------------
    u32x4 kreg[KLOADS];
    u32x4 vreg[4];
    auto load_tile = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int c = r * NTHREADS + tid;
            const int key = c / DCH, dc = c - (c / DCH) * DCH;
            const int j = k0 + key;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (j < Lk) v = *(const u32x4 *)(Kp + (int64_t)j * a.k_ss + dc * 8);
            kreg[r] = v;
        }
        if (tid < VUNITS) {
            const int dc = tid % DCH, kg = tid / DCH;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int j = k0 + kg * 4 + rr;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (j < Lk) v = *(const u32x4 *)(Vp + (int64_t)j * a.v_ss + dc * 8);
                vreg[rr] = v;
            }
        }
    };
    auto store_tile = [&](int stage) {
        unsigned short *Ks = smem + stage * STAGE;
        unsigned short *Vt = Ks + K_ELEMS;
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int c = r * NTHREADS + tid;
            const int key = c / DCH, dc = c - (c / DCH) * DCH;
            *(u32x4 *)(Ks + key * KS + dc * 8) = kreg[r];
        }
        if (tid < VUNITS) {
            const int dc = tid % DCH, kg = tid / DCH;
            const int key = kg * 4;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = e >> 1;
                unsigned lo, hi;
                if (e & 1) {
                    lo = (vreg[0][i] >> 16) | (vreg[1][i] & 0xffff0000u);
                    hi = (vreg[2][i] >> 16) | (vreg[3][i] & 0xffff0000u);
                } else {
                    lo = (vreg[0][i] & 0xffffu) | (vreg[1][i] << 16);
                    hi = (vreg[2][i] & 0xffffu) | (vreg[3][i] << 16);
                }
                const int d = dc * 8 + e;
                const int idx = d * BN + ((((key >> 3) ^ vt_swz(d)) << 3) | (key & 7));
                u32x2 w = {lo, hi};
                *(u32x2 *)(Vt + idx) = w;
            }
        }
    };

    f32x16 oacc[DBLK];
#pragma unroll
    for (int jd = 0; jd < DBLK; ++jd)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[jd][r] = 0.f;
    float m_run = -INFINITY;   // running row max, scaled log2 domain
    float l_run = 0.f;         // running row sum over this lane's keys

    if (t_begin < t_end) {
        load_tile(t_begin);
        store_tile(0);
    }
    __syncthreads();

    const int pos = qi + offset;                       // key position of this row
    const float c2 = a.scale_log2;

    for (int t = t_begin; t < t_end; ++t) {
        const int stage = (t - t_begin) & 1;
        const bool has_next = t + 1 < t_end;
        if (has_next) load_tile(t + 1);
        const unsigned short *Ks = smem + stage * STAGE;
        const unsigned short *Vt = Ks + K_ELEMS;
        const int k0 = t * BN;

        // S^T = K Q^T for two 32-key sub-blocks
        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
            const unsigned short *krow = Ks + (sb * 32 + perm32(l32)) * KS + half * 8;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const bf16x8 kf = *(const bf16x8 *)(krow + ks * 16);
                s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[sb], 0, 0, 0);
            }
        }

        // element mask, only on tiles that cross a boundary of this wave's rows
        const bool need_mask = (k0 + BN > Lk) ||
                               (a.causal && k0 + BN - 1 > q0w + offset) ||
                               (W > 0 && k0 <= q0w + 31 + offset - W);
        if (need_mask) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + sb * 32 + ((r >> 3) << 4) + half * 8 + (r & 7);
                    bool vis = key < Lk;
                    if (a.causal) vis = vis && key <= pos;
                    if (W > 0) vis = vis && key > pos - W;
                    if (!vis) s[sb][r] = -INFINITY;
                }
        }

        // online softmax update (fp32, base-2 exponent with scale folded in)
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * c2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        bf16x8 pb[2][2];
        float psum = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], c2, -m_use));
                psum += p[r];
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(p[tt * 8 + 2 * i], p[tt * 8 + 2 * i + 1]);
                pb[sb][tt] = __builtin_bit_cast(bf16x8, w);
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int jd = 0; jd < DBLK; ++jd)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[jd][r] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int jd = 0; jd < DBLK; ++jd) {
            const int d = jd * 32 + l32;
            const unsigned short *vrow = Vt + d * BN;
            const int sw = vt_swz(d);
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int chunk = sb * 4 + tt * 2 + half;
                    const bf16x8 vf = *(const bf16x8 *)(vrow + ((chunk ^ sw) << 3));
                    oacc[jd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[sb][tt], oacc[jd], 0, 0, 0);
                }
        }

        if (has_next) store_tile(stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: normalise once, write O (bf16, RNE) and LSE -------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool row_ok = qi < Lq && l_tot > 0.f;
    const float inv = row_ok ? 1.f / l_tot : 0.f;
    if (qi < a.seqlen_q) {
        unsigned short *orow = (unsigned short *)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_ss;
#pragma unroll
        for (int jd = 0; jd < DBLK; ++jd)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = jd * 32 + j * 8 + half * 4;
                u32x2 w;
                w[0] = pack_bf16x2(oacc[jd][4 * j] * inv, oacc[jd][4 * j + 1] * inv);
                w[1] = pack_bf16x2(oacc[jd][4 * j + 2] * inv, oacc[jd][4 * j + 3] * inv);
                *(u32x2 *)(orow + d) = w;
            }
        if (a.lse && half == 0) {
            float* lrow = a.lse + ((int64_t)b * a.heads_q + h) * a.seqlen_q;
            lrow[qi] = row_ok ? (m_run + log2f(l_tot)) * LN2 : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)a.num_q_tiles * a.heads_q * a.batch);
    const dim3 block(NTHREADS);
    if (head_dim == 128)
        hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace fa
