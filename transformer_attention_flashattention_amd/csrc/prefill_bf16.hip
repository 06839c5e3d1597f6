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
//   * KV tiles of 64 keys move HBM -> LDS with direct-to-LDS loads
//     (global_load_lds_dwordx4: no VGPR staging), double buffered: tile t+1
//     streams into one LDS buffer while tile t is computed from the other (the
//     two-region ping-pong of the hwcomputing.csdn.net page, section 2.1).
//   * the causal / window / valid-length masks are index arithmetic: tiles
//     wholly outside the visible band are never visited, and the element mask
//     runs only on tiles that cross a boundary (jsqmd.com page, section 二
//     "causal mask and decode").  Rows at or beyond the valid key length are
//     never read: their loads are redirected to the last valid row and the
//     corresponding scores are masked (agent.csdn.net BERT page, chapter 四).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, 64 lanes):
//   S^T[key][query] = K Q^T : A = K rows from LDS, B = Q held in registers.
//     Each lane holds one query column and 16 of the 32 keys of a sub-block,
//     so row max / row sum are lane-local except for one exchange with the
//     partner lane (lane ^ 32) holding the other 16 keys.
//   O^T[dim][query] += V^T P^T : B = P^T straight from the S^T accumulator
//     registers converted to bf16; A = V^T read from the row-major V tile with
//     the LDS transpose read ds_read_b64_tr_b16.  K rows are fetched in a
//     permuted order (bits 2 and 3 of the sub-block row swapped) so that each
//     lane's 8 consecutive accumulator registers hold 8 consecutive keys,
//     matching the key order the transpose read produces.
//   LDS tiles are unpadded rows with an XOR swizzle of 16-byte chunks (chosen
//   per tensor so that both the K operand reads and the V transpose reads are
//   free of bank conflicts); the swizzle is applied on the global side of the
//   direct loads, which always write 1 KiB contiguous per wavefront.
//
// Softmax bookkeeping: the row reference max only moves when the running max
// exceeds it by more than 2^8 (in the base-2 exponent domain); until then P
// is taken against the old reference, so O, the row sum and P always share
// one reference and the result is exact -- only the rescale work is skipped.
#include "fa_internal.h"

#include <climits>
#include <cmath>

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;

constexpr int BM = kPrefillBM;   // query rows per workgroup
constexpr int BN = 64;           // keys per KV tile
constexpr int NTHREADS = 256;
constexpr float LN2 = 0.693147180559945309f;
constexpr float RESCALE_THRESHOLD = 8.0f;   // log2 of the largest un-rescaled p

// Row permutation of a 32-key sub-block: swap bits 2 and 3.
__device__ __forceinline__ int perm32(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D>
struct Tile {
    static constexpr int ROWB = D * 2;           // bytes per row (unpadded)
    static constexpr int CH = D / 8;             // 16-byte chunks per row
    static constexpr int RPW = 256 / ROWB;       // rows per 256-byte LDS bank window
    static constexpr int BYTES = BN * ROWB;      // bytes per K or V tile
    static constexpr int LOADS_PER_WAVE = BYTES / 1024 / 4;
    // physical chunk of logical chunk c in row r
    __device__ static __forceinline__ int k_chunk(int r, int c) { return c ^ ((r / RPW) & (CH - 1)); }
    __device__ static __forceinline__ int v_chunk(int r, int c) {
        return c ^ ((((r / RPW) & 3) << 2) & (CH - 1));
    }
};

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ void wait_loads() {
    // vmcnt(0); expcnt and lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2)))
void prefill_bf16_kernel(PrefillArgs a) {
    using T = Tile<D>;
    constexpr int KSTEPS = D / 16;        // MFMA k-steps over head_dim for S
    constexpr int DBLK = D / 32;          // 32-dim row blocks of O^T

    __shared__ __attribute__((aligned(1024))) char sK0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char sV0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char sK1[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char sV1[T::BYTES];

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
    const int t_begin = kv_lo / BN;
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

    // ---- HBM -> LDS, one KV tile, 1 KiB per wavefront instruction ----------
    auto issue_tile = [&](int t, char *kb, char *vb) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
            const int ins = wave * T::LOADS_PER_WAVE + i;
            const int lin = ins * 1024 + lane * 16;
            const int r = lin / T::ROWB;
            const int p = (lin % T::ROWB) >> 4;
            const int row = min(k0 + r, Lk - 1);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(Kp + (int64_t)row * a.k_ss + T::k_chunk(r, p) * 8),
                (__attribute__((address_space(3))) void *)(kb + ins * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(Vp + (int64_t)row * a.v_ss + T::v_chunk(r, p) * 8),
                (__attribute__((address_space(3))) void *)(vb + ins * 1024), 16, 0, 0);
        }
    };

    f32x16 oacc[DBLK];
#pragma unroll
    for (int jd = 0; jd < DBLK; ++jd)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[jd][r] = 0.f;
    float m_ref = -INFINITY;   // reference row max, scaled log2 domain
    float l_run = 0.f;         // running row sum over this lane's keys

    const int pos = qi + offset;                       // key position of this row
    const float c2 = a.scale_log2;
    const int vis_hi = a.causal ? min(Lk, pos + 1) : Lk;
    const int vis_lo = (W > 0) ? pos - W + 1 : INT_MIN;

    // per-lane constant parts of the LDS operand addresses
    int k_row[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) k_row[sb] = sb * 32 + perm32(l32);
    const int g16 = lane >> 4, r16 = lane & 15;

    auto compute_tile = [&](int t, const char *kb, const char *vb) {
        const int k0 = t * BN;

        // S^T = K Q^T for two 32-key sub-blocks: all K fragments are read
        // first, then the two independent accumulation chains alternate.
        f32x16 s[2];
        bf16x8 kf[2][KSTEPS];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int r = k_row[sb];
            const char *krow = kb + r * T::ROWB;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                kf[sb][ks] = *(const bf16x8 *)(krow + (T::k_chunk(r, ks * 2 + half) << 4));
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2) s[sb][r2] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
                s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[sb][ks], qf[ks], s[sb], 0, 0, 0);

        // element mask (branch-free), only on tiles that cross a boundary of
        // this wave's rows: visible keys of this row are [vis_lo, vis_hi)
        const bool need_mask = (k0 + BN > Lk) ||
                               (a.causal && k0 + BN - 1 > q0w + offset) ||
                               (W > 0 && k0 <= q0w + 31 + offset - W);
        if (need_mask) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + sb * 32 + ((r >> 3) << 4) + half * 8 + (r & 7);
                    s[sb][r] = (key >= vis_lo && key < vis_hi) ? s[sb][r] : -INFINITY;
                }
        }

        // online softmax (fp32, base-2 exponent with the scale folded in)
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_ref, mx * c2);
        if (__ballot(m_new > m_ref + RESCALE_THRESHOLD)) {
            // move the reference: at least one row of this wave grew too far
            const float m_to = (m_new > m_ref + RESCALE_THRESHOLD) ? m_new : m_ref;
            // 1 for rows that keep their reference (also when both are -inf),
            // 0 when the old reference is -inf (nothing accumulated yet)
            const float alpha = (m_to == m_ref) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_to);
            m_ref = m_to;
            l_run *= alpha;
#pragma unroll
            for (int jd = 0; jd < DBLK; ++jd)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[jd][r] *= alpha;
        }
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;

        bf16x8 pb[4];
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
                pb[sb * 2 + tt] = __builtin_bit_cast(bf16x8, w);
            }
        }
        l_run += psum;

        // O^T += V^T P^T ; V^T operand from the row-major V tile by transpose
        // reads, all four key steps of a 32-dim block fetched before its MFMAs
#pragma unroll
        for (int jd = 0; jd < DBLK; ++jd) {
            const int c = 4 * jd + 2 * (g16 & 1) + ((r16 & 3) >> 1);
            const int byte_in_chunk = (r16 & 1) * 8;
            bf16x8 vf[4];
#pragma unroll
            for (int ksp = 0; ksp < 4; ++ksp) {
                s16x4 part[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int row = 16 * ksp + 8 * half + 4 * tt + (r16 >> 2);
                    const char *addr = vb + row * T::ROWB + (T::v_chunk(row, c) << 4) + byte_in_chunk;
                    part[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(addr));
                }
                typedef __attribute__((ext_vector_type(8))) short s16x8;
                const s16x8 both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
                vf[ksp] = __builtin_bit_cast(bf16x8, both);
            }
#pragma unroll
            for (int ksp = 0; ksp < 4; ++ksp)
                oacc[jd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ksp], pb[ksp], oacc[jd], 0, 0, 0);
        }
    };

    // ---- main loop: two statically named LDS buffers, unrolled by two -------
    if (t_begin < t_end) issue_tile(t_begin, sK0, sV0);
    wait_loads();
    __syncthreads();
    for (int t = t_begin; t < t_end; t += 2) {
        if (t + 1 < t_end) issue_tile(t + 1, sK1, sV1);
        compute_tile(t, sK0, sV0);
        wait_loads();
        __syncthreads();
        if (t + 1 < t_end) {
            if (t + 2 < t_end) issue_tile(t + 2, sK0, sV0);
            compute_tile(t + 1, sK1, sV1);
            wait_loads();
            __syncthreads();
        }
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
            float *lrow = a.lse + ((int64_t)b * a.heads_q + h) * a.seqlen_q;
            lrow[qi] = row_ok ? (m_ref + log2f(l_tot)) * LN2 : -INFINITY;
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
