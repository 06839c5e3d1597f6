// Single-token decode over a contiguous BSHD KV cache, bf16, for gfx950.
//
// The incremental mode of the agent.csdn.net BERT page (closing section):
// the new token's query attends to every cached key/value of its sequence;
// nothing already in the cache is recomputed.  The work is a stream over the
// cache, so the kernels are organised around HBM bandwidth, not MFMA:
//
// Split kernel -- one workgroup per (sequence, KV head, chunk of C keys):
//   * every K and V row of the chunk is read from HBM exactly once and used
//     for all query heads of its GQA group (query head h reads KV head
//     h / group);
//   * all of the chunk's K and V loads are issued up front as 16-byte vector
//     loads (8 or 16 lanes cover one 256-byte row, so each wavefront-wide
//     load instruction touches whole 128-byte segments), keeping many bytes
//     in flight per CU;
//   * scores q.k use the packed bf16 dot product (v_dot2_f32_bf16, fp32
//     accumulate) and a 3-step DPP reduction inside each 8-lane row group;
//   * the chunk's softmax statistics (max m, sum l, base-2 with the scale
//     folded in) and its unnormalised P.V are written to the workspace.
// Combine kernel -- one wavefront per (sequence, query head): merges the
//   chunk partials with the log-sum-exp rule (M = max m_c; L = sum 2^(m_c-M)
//   l_c; O = sum 2^(m_c-M) O_c / L; LSE = ln 2 (M + log2 L)), which is the
//   same max correction the running softmax uses within a chunk
//   (hwcomputing.csdn.net page, section 2.2), and writes O (bf16) and LSE.
#include "fa_internal.h"

#include <cmath>

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int NTHREADS = 256;
constexpr float LN2 = 0.693147180559945309f;

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the 8 lanes of an aligned group (every lane gets the total).
__device__ __forceinline__ float sum8(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    return x;
}

// Keys [lo, L) of sequence b are visible to its decode query.
__device__ __forceinline__ void visible_range(const DecodeArgs &a, int b, int &lo, int &L) {
    L = min(max(a.seqlens_k[b], 0), a.capacity);
    lo = (a.window_left > 0) ? max(0, L - a.window_left) : 0;
}

// D: head_dim; GT: query heads per workgroup; C: keys per chunk.
template <int D, int GT, int C>
__global__ __launch_bounds__(NTHREADS) void decode_split_kernel(DecodeArgs a) {
    constexpr int DPL = D / 8;               // dims per lane in the score phase (8 lanes / key)
    constexpr int KVEC = DPL / 8;            // 16-byte loads per key per lane (score phase)
    constexpr int KPASS = NTHREADS / 8;      // keys per pass in the score phase
    constexpr int NK = C / KPASS;            // keys per lane in the score phase
    constexpr int LV = D / 8;                // lanes per key in the value phase
    constexpr int VPASS = NTHREADS / LV;     // keys per pass in the value phase
    constexpr int NV = C / VPASS;            // keys per lane in the value phase
    static_assert(C % KPASS == 0 && C % VPASS == 0, "chunk size");

    __shared__ __attribute__((aligned(16))) float sc[C * GT];          // scores, then p
    __shared__ float red[2][NTHREADS / 64][GT];
    __shared__ __attribute__((aligned(16))) float ored[VPASS][GT][D];  // value-phase partials

    const int chunk = blockIdx.x;
    const int hg = blockIdx.y % a.head_groups;
    const int kvh = blockIdx.y / a.head_groups;
    const int b = blockIdx.z;
    int lo, L;
    visible_range(a, b, lo, L);
    const int c_lo = lo / C, c_hi = (L + C - 1) / C;
    if (chunk < c_lo || chunk >= c_hi) return;     // nothing visible in this chunk
    const int k0 = chunk * C;
    const int h0 = kvh * a.group + hg * GT;        // first query head of this workgroup

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const unsigned short *Kp = (const unsigned short *)a.k + b * a.k_sb + kvh * a.k_sh;
    const unsigned short *Vp = (const unsigned short *)a.v + b * a.v_sb + kvh * a.v_sh;

    // ---- issue every K and V load of the chunk ----------------------------
    const int ksub = tid & 7, kslot = tid >> 3;
    u32x4 kr[NK][KVEC];
#pragma unroll
    for (int p = 0; p < NK; ++p) {
        const int j = k0 + p * KPASS + kslot;
        const bool ok = j >= lo && j < L;
#pragma unroll
        for (int v = 0; v < KVEC; ++v) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (ok) x = *(const u32x4 *)(Kp + (int64_t)j * a.k_ss + v * 64 + ksub * 8);
            kr[p][v] = x;
        }
    }
    const int vsub = tid % LV, vslot = tid / LV;
    u32x4 vr[NV];
#pragma unroll
    for (int p = 0; p < NV; ++p) {
        const int j = k0 + p * VPASS + vslot;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (j >= lo && j < L) x = *(const u32x4 *)(Vp + (int64_t)j * a.v_ss + vsub * 8);
        vr[p] = x;
    }

    // ---- query slices for the score phase (bf16 pairs) --------------------
    unsigned qr[GT][KVEC][4];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        const unsigned short *qp = (const unsigned short *)a.q + b * a.q_sb + (h0 + g) * a.q_sh;
#pragma unroll
        for (int v = 0; v < KVEC; ++v) {
            const u32x4 x = *(const u32x4 *)(qp + v * 64 + ksub * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) qr[g][v][i] = x[i];
        }
    }

    // ---- scores ------------------------------------------------------------
#pragma unroll
    for (int p = 0; p < NK; ++p) {
        const int jl = p * KPASS + kslot;
        const int j = k0 + jl;
        const bool ok = j >= lo && j < L;
        float sg[GT];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float acc = 0.f;
#pragma unroll
            for (int v = 0; v < KVEC; ++v)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = dot2(kr[p][v][i], qr[g][v][i], acc);
            sg[g] = sum8(acc);
        }
        if (ksub == 0) {
#pragma unroll
            for (int g = 0; g < GT; ++g) sc[jl * GT + g] = ok ? sg[g] : -INFINITY;
        }
    }
    __syncthreads();

    // ---- chunk softmax statistics per head ---------------------------------
    // Thread t only ever touches entries of head t % GT.
    constexpr int PER = (C * GT + NTHREADS - 1) / NTHREADS;
    const int myg = tid % GT;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = i * NTHREADS + tid;
        if (idx < C * GT) mx = fmaxf(mx, sc[idx]);
    }
#pragma unroll
    for (int off = GT; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane < GT) red[0][wave][lane] = mx;
    __syncthreads();
    float m2 = red[0][0][myg];
#pragma unroll
    for (int w = 1; w < NTHREADS / 64; ++w) m2 = fmaxf(m2, red[0][w][myg]);
    m2 *= a.scale_log2;                                   // base-2, scaled
    const float m_use = (m2 == -INFINITY) ? 0.f : m2;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = i * NTHREADS + tid;
        if (idx < C * GT) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[idx], a.scale_log2, -m_use));
            sc[idx] = p;
            ls += p;
        }
    }
#pragma unroll
    for (int off = GT; off < 64; off <<= 1) ls += __shfl_xor(ls, off);
    if (lane < GT) red[1][wave][lane] = ls;
    __syncthreads();

    // ---- unnormalised P.V over the chunk -----------------------------------
    float o[GT][8];
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
#pragma unroll
    for (int p = 0; p < NV; ++p) {
        const int jl = p * VPASS + vslot;
        float pg[GT];
#pragma unroll
        for (int g = 0; g < GT; ++g) pg[g] = sc[jl * GT + g];
        float vf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vf[2 * i] = bf_lo(vr[p][i]);
            vf[2 * i + 1] = bf_hi(vr[p][i]);
        }
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[g][e] = __builtin_fmaf(pg[g], vf[e], o[g][e]);
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        *(float4 *)&ored[vslot][g][vsub * 8] = make_float4(o[g][0], o[g][1], o[g][2], o[g][3]);
        *(float4 *)&ored[vslot][g][vsub * 8 + 4] = make_float4(o[g][4], o[g][5], o[g][6], o[g][7]);
    }
    __syncthreads();

    // ---- reduce over key slots and write the chunk partial -----------------
    for (int idx = tid; idx < GT * D; idx += NTHREADS) {
        const int g = idx / D, d = idx - (idx / D) * D;
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < VPASS; ++s) acc += ored[s][g][d];
        const int64_t row = ((int64_t)b * a.heads_q + h0 + g) * a.max_chunks + chunk;
        a.ws_o[row * D + d] = acc;
    }
    if (tid < GT) {
        float mm = red[0][0][tid];
        float ll = red[1][0][tid];
#pragma unroll
        for (int w = 1; w < NTHREADS / 64; ++w) {
            mm = fmaxf(mm, red[0][w][tid]);
            ll += red[1][w][tid];
        }
        const int64_t row = ((int64_t)b * a.heads_q + h0 + tid) * a.max_chunks + chunk;
        a.ws_ml[row * 2 + 0] = mm * a.scale_log2;
        a.ws_ml[row * 2 + 1] = ll;
    }
}

// One workgroup of 4 wavefronts per (sequence, query head).  Every lane of
// every wavefront holds the (m, l) of one chunk (64 chunks per pass), so each
// wavefront derives the global max and all weights on its own; wavefront w
// then sums chunks w, w+4, w+8, ... with all of its partial-O loads issued
// before the first use, and the four partial sums meet in LDS.  Each
// (sequence, head) therefore costs about one memory round trip per 64 chunks.
constexpr int COMBINE_THREADS = 256;
constexpr int COMBINE_UNROLL = 16;   // chunks per wavefront per pass (64 / 4)

template <int D>
__global__ __launch_bounds__(COMBINE_THREADS) void decode_combine_kernel(DecodeArgs a) {
    constexpr int DPL = (D + 63) / 64;       // dims per lane
    __shared__ float part[COMBINE_THREADS / 64][D];
    __shared__ float lpart[COMBINE_THREADS / 64];

    const int bh = blockIdx.x;
    const int b = bh / a.heads_q, h = bh - (bh / a.heads_q) * a.heads_q;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int lo, L;
    visible_range(a, b, lo, L);
    const int C = a.chunk;
    const int c_lo = lo / C, c_hi = (L > lo) ? (L + C - 1) / C : c_lo;
    const int n = c_hi - c_lo;
    const int64_t base = ((int64_t)b * a.heads_q + h) * a.max_chunks + c_lo;

    float M = -INFINITY;
    for (int j = lane; j < n; j += 64) M = fmaxf(M, a.ws_ml[(base + j) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float M_use = (M == -INFINITY) ? 0.f : M;

    float acc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
    float Lsum = 0.f;
    for (int j0 = 0; j0 < n; j0 += 64) {
        // partial O rows of this wavefront's chunks in this pass: loads first
        float ov[COMBINE_UNROLL][DPL];
#pragma unroll
        for (int u = 0; u < COMBINE_UNROLL; ++u) {
            const int j = j0 + wave + 4 * u;
#pragma unroll
            for (int i = 0; i < DPL; ++i) {
                const int d = lane * DPL + i;
                ov[u][i] = (j < n && d < D) ? a.ws_o[(base + j) * D + d] : 0.f;
            }
        }
        const int jl = j0 + lane;
        float w = 0.f, lw = 0.f;
        if (jl < n) {
            w = __builtin_amdgcn_exp2f(a.ws_ml[(base + jl) * 2] - M_use);
            lw = w * a.ws_ml[(base + jl) * 2 + 1];
        }
        Lsum += lw;
#pragma unroll
        for (int u = 0; u < COMBINE_UNROLL; ++u) {
            const float wc = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), wave + 4 * u));
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc[i] = __builtin_fmaf(wc, ov[u][i], acc[i]);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Lsum += __shfl_xor(Lsum, off);
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
        const int d = lane * DPL + i;
        if (d < D) part[wave][d] = acc[i];
    }
    if (lane == 0) lpart[wave] = Lsum;
    __syncthreads();
    if (wave != 0) return;

    // every wavefront summed all chunk weights, so any lpart entry is the total
    const float Ltot = lpart[0];
    const bool ok = Ltot > 0.f;
    const float inv = ok ? 1.f / Ltot : 0.f;
    unsigned short *orow = (unsigned short *)a.o + b * a.o_sb + h * a.o_sh;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
        const int d = lane * DPL + i;
        if (d < D) {
            float v = part[0][d];
#pragma unroll
            for (int w2 = 1; w2 < COMBINE_THREADS / 64; ++w2) v += part[w2][d];
            const __bf16 x = (__bf16)(v * inv);
            orow[d] = __builtin_bit_cast(unsigned short, x);
        }
    }
    if (a.lse && lane == 0)
        a.lse[(int64_t)b * a.heads_q + h] = ok ? (M_use + log2f(Ltot)) * LN2 : -INFINITY;
}

template <int D, int GT>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid(a.max_chunks, a.heads_kv * a.head_groups, a.batch);
    switch (a.chunk) {
        case 64: hipLaunchKernelGGL((decode_split_kernel<D, GT, 64>), grid, dim3(NTHREADS), 0, s, a); break;
        case 128: hipLaunchKernelGGL((decode_split_kernel<D, GT, 128>), grid, dim3(NTHREADS), 0, s, a); break;
        default: hipLaunchKernelGGL((decode_split_kernel<D, GT, 256>), grid, dim3(NTHREADS), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_all(const DecodeArgs &a, int gt, hipStream_t s) {
    hipError_t e;
    switch (gt) {
        case 1: e = launch_split<D, 1>(a, s); break;
        case 2: e = launch_split<D, 2>(a, s); break;
        default: e = launch_split<D, 4>(a, s); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.batch * a.heads_q), dim3(COMBINE_THREADS), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, int head_dim, int heads_per_wg, hipStream_t s) {
    if (head_dim == 128) return launch_all<128>(a, heads_per_wg, s);
    return launch_all<64>(a, heads_per_wg, s);
}

}  // namespace fa
