// Rotary position encoding of K for the 16-bit (bf16 / half) prefill, for gfx950.
//
// RoPE (jsqmd.com ops-transformer practice page, section 三, rotary position
// encoding): the vector at position m is rotated pair by pair; each pair of
// adjacent dims (2p, 2p + 1), p < rotary_dim / 2, turns by its own angle,
// here given by the caller's tables cos[m, p] and sin[m, p]:
//   (x, y) -> (x c - y s, x s + y c).
// The bf16 prefill kernel reads every key tile once per 256 query rows, so
// rotating keys inside it would repeat the rotation that many times on the
// wavefronts that feed the matrix core.  Instead this pass rotates each key
// row once (key j at position j) into a contiguous copy that the attention
// kernel then reads; queries are rotated inside the attention kernel as they
// are loaded.  The pass streams K once, one thread per 16-byte piece (8 dims,
// 4 pairs) at a time.
// Rows at or beyond a sequence's valid key length are neither read nor
// written (the attention kernel never reads them either).
#include "fa_internal.h"

#include <type_traits>

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// Rotate one adjacent pair held as two 16-bit values (bf16, or half with
// F16), rounding the result back to that type.
template <bool F16>
__device__ __forceinline__ unsigned rotate_pair(unsigned xy, float c, float s) {
    using v2 = typename std::conditional<F16, f16x2, bf16x2>::type;
    using et = typename std::conditional<F16, _Float16, __bf16>::type;
    const v2 v = __builtin_bit_cast(v2, xy);
    const float x = (float)v[0], y = (float)v[1];
    v2 r;
    r[0] = (et)__builtin_fmaf(x, c, -y * s);
    r[1] = (et)__builtin_fmaf(x, s, y * c);
    return __builtin_bit_cast(unsigned, r);
}

// Threads walk the rotated copy in its memory order: 16-byte pieces of whole
// key rows across all KV heads of a sequence (piece fastest, then head, then
// key), PER_THREAD pieces per thread spaced a workgroup apart, so loads and
// stores cover contiguous runs of rows in the BSHD layout and the heads of a
// row share their cos / sin entries in the caches.
constexpr int ROPE_THREADS = 256;
constexpr int ROPE_PER_THREAD = 4;

template <int D, bool F16>
__global__ __launch_bounds__(ROPE_THREADS) void rope_k_bf16_kernel(RopeKArgs a) {
    constexpr int PIECES = D / 8;                        // 16-byte pieces per head row
    const int b = blockIdx.y;
    const int Lk = a.seqlens_k ? min(max(a.seqlens_k[b], 0), a.seqlen_k) : a.seqlen_k;
    const int64_t row_pieces = (int64_t)a.heads_kv * PIECES;
    const int64_t n_end = (int64_t)Lk * row_pieces;      // pieces of the valid rows
    const int half = a.rotary_dim / 2;
    const int64_t n0 = (int64_t)blockIdx.x * ROPE_THREADS * ROPE_PER_THREAD + threadIdx.x;
#pragma unroll
    for (int u = 0; u < ROPE_PER_THREAD; ++u) {
        const int64_t n = n0 + (int64_t)u * ROPE_THREADS;
        if (n >= n_end) break;
        const int piece = (int)(n % PIECES);
        const int64_t r = n / PIECES;
        const int kvh = (int)(r % a.heads_kv);
        const int j = (int)(r / a.heads_kv);
        const unsigned short *src =
            (const unsigned short *)a.k + b * a.k_sb + (int64_t)j * a.k_ss + kvh * a.k_sh + piece * 8;
        u32x4 v = *(const u32x4 *)src;
        if (piece * 8 < a.rotary_dim) {                  // rotary_dim is a multiple of 8
            const float4 c = *(const float4 *)(a.rope_cos + (int64_t)j * half + piece * 4);
            const float4 sn = *(const float4 *)(a.rope_sin + (int64_t)j * half + piece * 4);
            v[0] = rotate_pair<F16>(v[0], c.x, sn.x);
            v[1] = rotate_pair<F16>(v[1], c.y, sn.y);
            v[2] = rotate_pair<F16>(v[2], c.z, sn.z);
            v[3] = rotate_pair<F16>(v[3], c.w, sn.w);
        }
        unsigned short *dst = (unsigned short *)a.out + ((int64_t)b * a.seqlen_k * a.heads_kv + r) * D + piece * 8;
        *(u32x4 *)dst = v;
    }
}

}  // namespace

hipError_t launch_rope_k_bf16(const RopeKArgs &a, int head_dim, bool f16, hipStream_t s) {
    const int64_t pieces = (int64_t)a.seqlen_k * a.heads_kv * (head_dim / 8);
    const int64_t per_wg = (int64_t)ROPE_THREADS * ROPE_PER_THREAD;
    const dim3 grid((unsigned)((pieces + per_wg - 1) / per_wg), (unsigned)a.batch);
    if (f16) {
        if (head_dim == 128) hipLaunchKernelGGL((rope_k_bf16_kernel<128, true>), grid, dim3(ROPE_THREADS), 0, s, a);
        else hipLaunchKernelGGL((rope_k_bf16_kernel<64, true>), grid, dim3(ROPE_THREADS), 0, s, a);
    } else {
        if (head_dim == 128) hipLaunchKernelGGL((rope_k_bf16_kernel<128, false>), grid, dim3(ROPE_THREADS), 0, s, a);
        else hipLaunchKernelGGL((rope_k_bf16_kernel<64, false>), grid, dim3(ROPE_THREADS), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace fa
