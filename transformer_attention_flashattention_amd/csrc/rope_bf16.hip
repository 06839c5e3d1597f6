// Rotary position encoding of K for the bf16 prefill, for gfx950.
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
// are loaded.  The pass streams K once: one thread per 16-byte piece (8 dims,
// 4 pairs) of a row, a grid-stride loop over [batch, key, KV head, piece].
// Rows at or beyond a sequence's valid key length are neither read nor
// written (the attention kernel never reads them either).
#include "fa_internal.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ unsigned rotate_pair(unsigned xy, float c, float s) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, xy);
    const float x = (float)v[0], y = (float)v[1];
    bf16x2 r;
    r[0] = (__bf16)__builtin_fmaf(x, c, -y * s);
    r[1] = (__bf16)__builtin_fmaf(x, s, y * c);
    return __builtin_bit_cast(unsigned, r);
}

template <int D>
__global__ __launch_bounds__(256) void rope_k_bf16_kernel(RopeKArgs a) {
    constexpr int PIECES = D / 8;
    const int half = a.rotary_dim / 2;
    const int64_t total = (int64_t)a.batch * a.seqlen_k * a.heads_kv * PIECES;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int piece = (int)(idx % PIECES);
        int64_t row = idx / PIECES;                      // (b, j, kvh) in BSHD order
        const int kvh = (int)(row % a.heads_kv);
        row /= a.heads_kv;
        const int j = (int)(row % a.seqlen_k);
        const int b = (int)(row / a.seqlen_k);
        const int Lk = a.seqlens_k ? min(max(a.seqlens_k[b], 0), a.seqlen_k) : a.seqlen_k;
        if (j >= Lk) continue;
        const unsigned short *src = (const unsigned short *)a.k + b * a.k_sb + (int64_t)j * a.k_ss +
                                    kvh * a.k_sh + piece * 8;
        u32x4 v = *(const u32x4 *)src;
        if (piece * 8 < a.rotary_dim) {                  // rotary_dim is a multiple of 8
            const float4 c = *(const float4 *)(a.rope_cos + (int64_t)j * half + piece * 4);
            const float4 s = *(const float4 *)(a.rope_sin + (int64_t)j * half + piece * 4);
            v[0] = rotate_pair(v[0], c.x, s.x);
            v[1] = rotate_pair(v[1], c.y, s.y);
            v[2] = rotate_pair(v[2], c.z, s.z);
            v[3] = rotate_pair(v[3], c.w, s.w);
        }
        *(u32x4 *)((unsigned short *)a.out + idx * 8) = v;
    }
}

}  // namespace

hipError_t launch_rope_k_bf16(const RopeKArgs &a, int head_dim, hipStream_t s) {
    const int64_t pieces = (int64_t)a.batch * a.seqlen_k * a.heads_kv * (head_dim / 8);
    const int64_t want = (pieces + 255) / 256;
    const unsigned blocks = (unsigned)(want < 16384 ? (want > 0 ? want : 1) : 16384);
    if (head_dim == 128) hipLaunchKernelGGL(rope_k_bf16_kernel<128>, dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(rope_k_bf16_kernel<64>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace fa
