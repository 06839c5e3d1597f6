// Single-token decode over a contiguous BSHD KV cache, bf16, for gfx950.
//
// The incremental mode of the agent.csdn.net BERT page (closing section):
// the new token's query attends to every cached key/value of its sequence;
// nothing already in the cache is recomputed.  The work is a stream over the
// cache, so the kernels are organised around HBM bandwidth, not MFMA:
//
// Split kernel -- one workgroup (4 wavefronts) per (sequence, KV head, chunk
// of keys).  Every K and V row of the chunk is read from HBM exactly once and
// used for all query heads of its GQA group (query head h reads KV head
// h / group).  Each wavefront walks its share of the chunk in tiles of KT keys
// (wavefront w takes tiles w, w+4, ...) and keeps the next NBUF-1 tiles' K and
// V loads in flight (non-temporal 16-byte loads covering contiguous pieces of
// each row) while it computes the current one, with its own running softmax:
//   * scores: 16 dims per lane (two 16-byte pieces, each load instruction
//     covering contiguous half rows), packed bf16 dot products (v_dot2_f32_bf16,
//     fp32 accumulate) and a DPP sum over the lanes of a key;
//   * running max per head, kept as a reference that only moves when a tile
//     max passes it by 2^8 (base-2, scale folded in), so the accumulators are
//     rescaled only then (the max correction of the hwcomputing.csdn.net page,
//     section 2.2);
//   * P leaves the score layout through a KT x heads slot of LDS private to
//     the wavefront and is read back in the value layout (8 dims per lane),
//     where P.V accumulates in fp32 registers (packed bf16 dot products over
//     pairs of keys; P enters that product in bf16, its row sum in fp32).
// The four wavefronts merge their (max, sum, P.V) once per chunk through LDS
// and write the chunk's partial to the workspace.  With an FP8 cache both
// products run on the matrix cores instead (see decode_split below).
// Combine kernel -- one wavefront per (sequence, query head): merges the
//   chunk partials with the log-sum-exp rule (M = max m_c; L = sum 2^(m_c-M)
//   l_c; O = sum 2^(m_c-M) O_c / L; LSE = ln 2 (M + log2 L)), the same max
//   correction the running softmax uses within a chunk, and writes O (bf16)
//   and LSE.
#include "fa_internal.h"

#include <cmath>
#include <type_traits>

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int NTHREADS = 256;
constexpr int NWAVES = NTHREADS / 64;
constexpr int NBUF = 2;                      // tiles held in registers: 1 computing, 1 in flight
constexpr float LN2 = 0.693147180559945309f;
constexpr float RESCALE_THRESHOLD = 8.0f;    // log2 of the largest un-rescaled p


__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the N lanes (N = 4 or 8) of an aligned group; every lane gets the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);       // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);       // quad_perm [2,3,0,1]
    if constexpr (N == 8) x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    return x;
}

// Values of lanes l ^ 16 and l ^ 32, exchanged with the VALU lane swaps.
__device__ __forceinline__ float xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    // lanes of even rows find the partner in the second result, odd rows in the first
    return __builtin_bit_cast(float, (unsigned)(((threadIdx.x >> 4) & 1) ? r[0] : r[1]));
}
__device__ __forceinline__ float xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)(((threadIdx.x >> 5) & 1) ? r[0] : r[1]));
}
// Value of lane l ^ 8 (DPP row_ror:8 inside each row of 16 lanes).
__device__ __forceinline__ float xor8(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}
// Value of lane (l + 4) mod 16 inside each row of 16 lanes (DPP row_ror:4).
__device__ __forceinline__ float ror4(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
}
// Max / sum over the lanes that share l % N (N = 4 or 8): the lane groups of
// one key position in a layout with N lanes per key.
template <int N>
__device__ __forceinline__ float across_groups_max(float x) {
    if constexpr (N == 4) x = fmaxf(x, ror4(x));
    x = fmaxf(x, xor8(x));
    x = fmaxf(x, xor16(x));
    return fmaxf(x, xor32(x));
}
template <int N>
__device__ __forceinline__ float across_groups_sum(float x) {
    if constexpr (N == 4) x += ror4(x);
    x += xor8(x);
    x += xor16(x);
    return x + xor32(x);
}

// Max / sum over the 16 lanes of each row (DPP inside the row); every lane of
// the row gets the result.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false));      // quad_perm [1,0,3,2]
    x = fmaxf(x, __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false));      // quad_perm [2,3,0,1]
    x = fmaxf(x, __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false));     // row_half_mirror
    return fmaxf(x, __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xF, 0xF, false));  // row_mirror
}
__device__ __forceinline__ float row_sum16(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);
    return x + __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xF, 0xF, false);
}

// Keys [lo, L) of sequence b are visible to its decode query.
__device__ __forceinline__ int visible_lo(const DecodeArgs &a, int L) {
    return (a.window_left > 0) ? max(0, L - a.window_left) : 0;
}
__device__ __forceinline__ void visible_range(const DecodeArgs &a, int b, int &lo, int &L) {
    L = min(max(a.seqlens_k[b], 0), a.capacity);
    lo = visible_lo(a, L);
}

// First key of the chunk grid: lo rounded down to a multiple of a.origin_align (1 for a
// contiguous cache; the tile length for a paged cache, so that every tile
// lies inside one page).  Both kernels of a call use the same value.
__device__ __forceinline__ int chunk_origin(const DecodeArgs &a, int lo) {
    return lo & ~(a.origin_align - 1);            // origin_align: 1, 16 or 32
}

// The keys [origin, L) of a sequence are cut into n = ceil((L - origin) /
// a.chunk) chunks of equal length len (a multiple of 128, at most a.chunk);
// chunk c covers [origin + c len, min(L, origin + (c + 1) len)) and holds a
// visible key (origin > lo - 128).  Equal chunks keep the workgroups of one
// sequence equally long.
__device__ __forceinline__ void chunking(const DecodeArgs &a, int lo, int L, int &n, int &len) {
    const int Lv = L - chunk_origin(a, lo);
    n = (Lv + a.chunk - 1) / a.chunk;
    len = n > 0 ? (((Lv + n - 1) / n + kDecodeChunkUnit - 1) / kDecodeChunkUnit) * kDecodeChunkUnit : 0;
}

// Work items are the (sequence, chunk) pairs that exist.  They are numbered
// block by block, 64 sequences to a block, and within a block longest chunk
// first (ties by sequence index, a sequence's chunks together), so the last
// workgroups of a launch are its shortest.  For the sequences b0 + lane of
// one block (a whole wavefront takes part): n = this lane's chunk count,
// ahead = items of the block that come before this lane's first, total =
// items of the block, L = this lane's valid length.
__device__ __forceinline__ void rank_block(const DecodeArgs &a, int b0, int lane, int &n, int &ahead,
                                           int &total, int &L) {
    int len = 0;
    n = 0;
    L = 0;
    if (b0 + lane < a.batch) {
        int lo;
        visible_range(a, b0 + lane, lo, L);
        chunking(a, lo, L, n, len);
    }
    // One key orders the lanes: chunk lengths are multiples of 128, so len / 2
    // is a multiple of 64 and the lane term (63 - lane) only breaks ties.
    static_assert(kDecodeChunkUnit % 128 == 0, "the order key needs len / 2 to be a multiple of 64");
    const int key = (len >> 1) + (63 - lane);
    ahead = 0;
    total = 0;
#pragma unroll
    for (int k = 0; k < 64; ++k) {
        const int key_k = __builtin_amdgcn_readlane(key, k);
        const int n_k = __builtin_amdgcn_readlane(n, k);
        ahead += key_k > key ? n_k : 0;
        total += n_k;
    }
}

// A buffer the launch only reads, seen through the constant address space:
// uniform loads from it become scalar loads whose waits the compiler tracks
// itself (through a generic pointer they become flat loads, and waiting for
// one of those also waits for every K/V load in flight).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T *read_only(const T *p) {
    return (const __attribute__((address_space(4))) T *)p;
}

template <typename T = u32x4>
__device__ __forceinline__ T load_nt(const char *base, unsigned off) {
    return __builtin_nontemporal_load((const T *)(base + off));
}

// The 16-bit type of q, o and of P in the P.V products: bf16, or IEEE half
// with F16.  Pairs of values travel packed in one 32-bit register.
template <bool F16> struct H16;
template <> struct H16<false> {
    using t = __bf16;
    static __device__ __forceinline__ unsigned pack(float lo, float hi) { return pack_bf16x2(lo, hi); }
    static __device__ __forceinline__ float dot(unsigned a, unsigned b, float c) { return dot2(a, b, c); }
    static __device__ __forceinline__ float lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
    static __device__ __forceinline__ float hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
    // two FP8 E4M3 codes (bytes 0-1 of w, or 2-3 with HI) as a pair; every
    // E4M3 value is exact in bf16
    template <bool HI>
    static __device__ __forceinline__ unsigned from_e4m3(unsigned w) {
        return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    }
    // 16 x 16 x 32 matrix product, fp32 accumulate
    static __device__ __forceinline__ f32x4 mma(u32x4 x, u32x4 y, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    }
};
template <> struct H16<true> {
    using t = _Float16;
    static __device__ __forceinline__ unsigned pack(float lo, float hi) {
        f16x2 r;
        r[0] = (_Float16)lo;
        r[1] = (_Float16)hi;
        return __builtin_bit_cast(unsigned, r);
    }
    static __device__ __forceinline__ float dot(unsigned a, unsigned b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    }
    static __device__ __forceinline__ float lo(unsigned w) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(unsigned w) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
    }
    // every E4M3 value is exact in half too (normal range 2^-6 .. 448,
    // subnormals down to 2^-9)
    template <bool HI>
    static __device__ __forceinline__ unsigned from_e4m3(unsigned w) {
        return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
    }
    static __device__ __forceinline__ f32x4 mma(u32x4 x, u32x4 y, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                      __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
    }
};

// D: head_dim; GT: query heads per workgroup (all of one KV head's group, or
// a slice of it); ALIBI: add the per-head linear bias -m (L - 1 - j); PAGED:
// the cache is a pool of pages named by a block table; KV8: K and V are FP8
// E4M3 codes with one scale per KV head each.  Chunk lengths are multiples of
// NWAVES * KT.  KT: keys per wavefront tile.  F16: q and o are IEEE half
// (and so is P in the P.V products) instead of bf16.
//
// With an FP8 cache the scores come from the matrix cores instead: per 16
// keys, D / 32 products v_mfma_f32_16x16x32 of Q (rows: the GT query heads,
// the other rows zero) with K^T (columns: the 16 keys), K's codes converted
// to bf16 in registers.  The product wants lane l to hold key l % 16 and the
// dims at 64 p + 16 (l / 16) .. +16 (p < D / 64); Q's operand holds the same
// dims of head l % 16 (a dot product may sum its dims in any order, so the
// same dims on both sides is all it needs).  Loaded that way, each load
// instruction would cover 64-byte pieces of 16 rows, which stream markedly
// slower than whole rows; so K is loaded in whole rows, as for the vector
// path, and each wavefront passes its tile through a private LDS slot (16-byte
// chunks XOR-swizzled by key) to read it back in the product's layout.
// Lanes 0-15 then hold the GT scores of their key; the vector path's dot
// products and lane sums per key (the bulk of its instructions) are gone.
// With 32-key tiles P.V goes to the matrix cores as well: O^T (D dims x the
// heads) += V^T P^T, D / 16 products of 16 dims x 32 keys.  V passes through
// a second LDS slot (rows as loaded, 16-byte chunks swizzled by key) and
// comes back through the 8-bit transpose read ds_read_b64_tr_b8: in each
// group of 16 lanes, lane i addresses 8 bytes of row i / 2 of an 8-row x
// 16-byte block and receives column i of its 8 rows, i.e. one dim of 8
// consecutive keys, the operand row the product wants.  P^T comes from LDS
// in head-major order (8 consecutive keys of head l % 16 per lane).  Lane l
// then holds O^T of dims 16 mm + 4 (l / 16) .. +4 for head l % 16.
template <int D, int GT, bool ALIBI, bool PAGED, bool KV8, int KT, bool F16>
__device__ __forceinline__ void decode_split(DecodeArgs a) {
    using H = H16<F16>;
    constexpr int SL = D / 16;               // score layout: lanes per key (16 dims each)
    constexpr int SKP = 64 / SL;             // keys per score pass
    constexpr int SP = KT / SKP;             // score passes per tile
    constexpr int VL = D / 8;                // value layout: lanes per key (8 dims each)
    constexpr int VKP = 64 / VL;             // keys per value pass
    constexpr int VP = KT / VKP;             // value passes per tile
    static_assert(GT <= SL && (SL == 4 || SL == 8), "layout");
    constexpr bool QKM = KV8;                // scores on the matrix cores (FP8 cache)
    constexpr int NM = D / 32;               // QKM: products per 16 keys
    constexpr int NG = KT / 16;              // QKM: 16-key groups per tile
    static_assert(!QKM || (KT % 16 == 0 && GT <= 4 && D % 64 == 0), "matrix-core score layout");
    constexpr bool PVM = QKM && KT == 32;    // P.V on the matrix cores too (32-key tiles)
    constexpr int ND = D / 16;               // PVM: products per tile (16 dims each)
    static_assert(kDecodeChunkUnit % (NWAVES * KT) == 0, "chunks hold whole tile rounds");

    __shared__ __attribute__((aligned(16))) float pw[NWAVES][KT][GT];   // P, per wavefront
    constexpr int CH = D / 16;                                           // 16-byte chunks of an FP8 row
    __shared__ u32x4 kst[QKM ? NWAVES : 1][QKM ? KT * CH : 1];          // QKM: K tile, per wavefront
    __shared__ u32x4 vst[PVM ? NWAVES : 1][PVM ? KT * CH : 1];          // PVM: V tile, per wavefront
    __shared__ __attribute__((aligned(16))) float pwt[PVM ? NWAVES : 1][GT][PVM ? KT : 1];  // PVM: P, head-major
    __shared__ __attribute__((aligned(16))) float mo[NWAVES][GT][D];    // merge: P.V
    __shared__ float mml[NWAVES][GT][2];                                 // merge: (m, l)

    // Each work item (see rank_block) is taken by heads_kv * head_groups
    // consecutive workgroups: KV head (group slice) varies fastest, so
    // workgroups dispatched together read the rows of all KV heads of one
    // key range (interleaved in the BSHD cache).  The grid is sized for
    // every sequence at capacity; workgroups past the last item exit.  Up to
    // 64 sequences (one block) each workgroup ranks the block itself; larger
    // batches read their item from the table decode_plan_kernel wrote.
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int slots = a.heads_kv * a.head_groups;
    const int item = blockIdx.x / slots;
    const int slot = blockIdx.x - item * slots;
    const int hg = slot % a.head_groups;
    const int kvh = slot / a.head_groups;
    int b = -1, chunk = 0, L = 0;
    if (a.ws_items) {
        const auto *items = read_only(a.ws_items);
        if (item < items[0]) {
            const int e = items[1 + item];
            b = e / a.max_chunks;
            chunk = e - b * a.max_chunks;
        }
        if (b < 0) return;                         // past the last work item
        b = __builtin_amdgcn_readfirstlane(b);
        chunk = __builtin_amdgcn_readfirstlane(chunk);
        L = min(max(a.seqlens_k[b], 0), a.capacity);
    } else {
        int n, ahead, total, L_lane;
        rank_block(a, 0, lane, n, ahead, total, L_lane);
        const unsigned long long hit = __ballot(n > 0 && item >= ahead && item < ahead + n);
        if (!hit) return;                          // past the last work item
        b = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
        chunk = item - __builtin_amdgcn_readlane(ahead, b);
        L = __builtin_amdgcn_readlane(L_lane, b);  // the length the ranking read
    }
    int nchunks, C;
    const int lo = visible_lo(a, L);
    chunking(a, lo, L, nchunks, C);
    const int k0 = chunk_origin(a, lo) + chunk * C;
    const int h0 = kvh * a.group + hg * GT;        // first query head of this workgroup
    // visible keys this workgroup owns (never empty)
    const int jlo = max(k0, lo), jhi = min(L, k0 + C);

    // wavefront index, made provably uniform so that branches on it are scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // contiguous cache: the sequence's rows of this KV head (paged: the
    // pool's page 0, replaced per tile)
    constexpr int ES = KV8 ? 1 : 2;                    // bytes per cached element
    const char *Kp = (const char *)a.k + ((PAGED ? 0 : b * a.k_sb) + kvh * a.k_sh) * ES;
    const char *Vp = (const char *)a.v + ((PAGED ? 0 : b * a.v_sb) + kvh * a.v_sh) * ES;
    // row offsets within one sequence (one page) fit 32 bits (checked on the host)
    const unsigned k_row = (unsigned)a.k_ss * ES, v_row = (unsigned)a.v_ss * ES;
    const int s_key = lane / SL, s_sub = lane % SL;    // score layout
    const int v_key = lane / VL, v_sub = lane % VL;    // value layout
    const int my_g = s_sub < GT ? s_sub : 0;           // head whose P this lane produces

    // query slice of every head, the same 16 dims a lane holds of each key
    // (8 bf16 pairs): bf16 keys, dims 8 s_sub .. +8 and D/2 + 8 s_sub .. +8
    // (each key load instruction then covers one contiguous half of every
    // row); FP8 keys, dims 16 s_sub .. +16 (one 16-byte load per row piece)
    // (matrix-core scores: qr[m] is product m's operand, 8 dims of head
    // qrow = l % 16 starting at qm_dim(m); zero for rows past GT)
    const int qrow = lane & 15, qgrp = lane >> 4;
    auto qm_dim = [&](int m) { return 64 * (m >> 1) + 16 * qgrp + 8 * (m & 1); };
    constexpr int QA = QKM ? NM : GT, QB = QKM ? 4 : 8;
    unsigned qr[QA][QB];
    if constexpr (QKM) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < GT)
                x = *(const u32x4 *)((const unsigned short *)a.q + b * a.q_sb + (h0 + qrow) * a.q_sh
                                     + qm_dim(m));
#pragma unroll
            for (int i = 0; i < 4; ++i) qr[m][i] = x[i];
        }
    } else {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const unsigned short *qp = (const unsigned short *)a.q + b * a.q_sb + (h0 + g) * a.q_sh
                                       + s_sub * 8;
            const u32x4 x0 = *(const u32x4 *)qp, x1 = *(const u32x4 *)(qp + D / 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qr[g][i] = x0[i];
                qr[g][4 + i] = x1[i];
            }
        }
    }

    // RoPE: the query sits at position L - 1 (L >= 1 for every work item);
    // each u32 of qr is one adjacent pair of dims, turned by its angle and
    // rounded back to bf16 (cached keys are stored already rotated)
    if (a.rotary_dim > 0) {
        const int rhalf = a.rotary_dim / 2;
        const float *cr = a.rope_cos + (int64_t)(L - 1) * rhalf;
        const float *sr = a.rope_sin + (int64_t)(L - 1) * rhalf;
        auto turn = [&](unsigned &w, int pr) __attribute__((always_inline)) {
            const float c = cr[pr], sn = sr[pr];
            const float x = H::lo(w), y = H::hi(w);
            w = H::pack(__builtin_fmaf(x, c, -y * sn), __builtin_fmaf(x, sn, y * c));
        };
        if constexpr (QKM) {
            if (qrow < GT) {
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        if (qm_dim(m) / 2 + w < rhalf) turn(qr[m][w], qm_dim(m) / 2 + w);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int pr = k < 4 ? 4 * s_sub + k : D / 4 + 4 * s_sub + (k - 4);
                if (pr < rhalf) {
#pragma unroll
                    for (int g = 0; g < GT; ++g) turn(qr[g][k], pr);
                }
            }
        }
    }

    // running state (m, the reference, is uniform across the wavefront)
    float m_ref[GT], o[GT][8];
    f32x4 ot[PVM ? ND : 1];                            // PVM: O^T of this lane's dims and head
#pragma unroll
    for (int mm = 0; mm < (PVM ? ND : 1); ++mm) ot[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    float l_part = 0.f;                                // this lane's share of the sum of head my_g
    float l_acc[GT];                                   // QKM: this lane's share of every head's sum
#pragma unroll
    for (int g = 0; g < GT; ++g) l_acc[g] = 0.f;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        m_ref[g] = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
    }
    const float c2 = a.scale_log2;
    // ALiBi in raw score units (see the prefill kernel): s - (m / scale) (L - 1 - j)
    float alibi_raw[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) alibi_raw[g] = ALIBI ? -a.alibi[h0 + g] / a.scale : 0.f;
    // FP8 cache: the per-KV-head scales (K's multiplies the raw dot product,
    // V's the partial P.V)
    const float k_scale = KV8 ? read_only(a.k_scale)[kvh] : 1.f;
    const float v_scale = KV8 ? read_only(a.v_scale)[kvh] : 1.f;

    // This wavefront's tiles t = 0, 1, ... start at key base + STEP t (STEP =
    // NWAVES * KT); the ones holding a visible key form one contiguous range
    // [ta, tb).
    constexpr int STEP = NWAVES * KT;
    const int ntl = C / STEP;
    const int base = k0 + wave * KT;
    auto tile_key0 = [&](int t) { return base + t * STEP; };
    auto cdiv = [](int n) { return n <= 0 ? -((-n) / STEP) : (n + STEP - 1) / STEP; };
    const int ta = max(0, cdiv(jlo - (KT - 1) - base));
    const int tb = min(ntl, cdiv(jhi - base));
    // Keys outside [jlo, jhi) load a clamped, valid row instead (finite data;
    // the score mask then gives them p = 0), so every load is unconditional and
    // the compiler can wait for exactly the current tile's loads.
    //
    // Paged cache: a tile starts at a multiple of KT keys (chunk_origin) and a
    // page holds a multiple of KT rows, so the keys of a tile share one page,
    // and so do their clamped stand-ins: they are jlo or jhi - 1, which lie in
    // the tile whenever any of its keys is visible, and otherwise every key of
    // the tile clamps to the same one.  That page is the page of the tile's
    // first key clamped to [jlo, jhi); the wavefront reads its table entry
    // (one uniform load) and addresses the rows inside it.
    // K: two 16-byte pieces per lane and pass (bf16) or one (FP8); V: 8 dims
    // per lane, 16 bytes (bf16) or 8 bytes (FP8)
    constexpr int KA = SP, KB = KV8 ? 1 : 2;
    using VVec = typename std::conditional<KV8, u32x2, u32x4>::type;
    u32x4 kb[NBUF][KA][KB];
    VVec vb[NBUF][VP];
    auto load = [&](int t, u32x4 (&kt)[KA][KB], VVec (&vt)[VP]) __attribute__((always_inline)) {
        const int t0 = tile_key0(t);
        const char *kbase = Kp, *vbase = Vp;
        int row0 = 0;                                  // logical key of row 0 at kbase
        if constexpr (PAGED) {
            const int anchor = min(max(t0, jlo), jhi - 1);
            const int pg = anchor / a.page_size;
            int phys = read_only(a.block_table)[(int64_t)b * a.pages_per_seq + pg];
            phys = min(max(phys, 0), a.num_pages - 1);
            kbase = Kp + (int64_t)phys * a.k_sb * ES;
            vbase = Vp + (int64_t)phys * a.v_sb * ES;
            row0 = pg * a.page_size;
        }
#pragma unroll
        for (int p = 0; p < SP; ++p) {
            const int j = min(max(t0 + p * SKP + s_key, jlo), jhi - 1);
            // each load instruction covers one contiguous half of every row it
            // touches (bf16) or whole rows (FP8)
            const unsigned off = (unsigned)(j - row0) * k_row + s_sub * 16;
            kt[p][0] = load_nt(kbase, off);
            if constexpr (!KV8) kt[p][1] = load_nt(kbase, off + D);
        }
#pragma unroll
        for (int p = 0; p < VP; ++p) {
            const int j = min(max(t0 + p * VKP + v_key, jlo), jhi - 1);
            vt[p] = load_nt<VVec>(vbase, (unsigned)(j - row0) * v_row + v_sub * 8 * ES);
        }
    };
    auto compute = [&](int t, const u32x4 (&kt)[KA][KB], const VVec (&vt)[VP]) __attribute__((always_inline)) {
        const int t0 = tile_key0(t);
        // scores for every head: of this lane's key in each score pass
        // (vector path), or of key l % 16 of each 16-key group (matrix path,
        // meaningful in lanes 0-15)
        float s[KA][GT];
        if constexpr (QKM) {
            // the tile's rows into the wavefront's slot (lane: chunk s_sub of
            // key p * SKP + s_key), chunk c of key k at c ^ (k % CH)
#pragma unroll
            for (int p = 0; p < SP; ++p) {
                const int k = p * SKP + s_key;
                kst[wave][k * CH + (s_sub ^ (k & (CH - 1)))] = kt[p][0];
            }
            if constexpr (PVM) {
                // V rows likewise (lane: 8 bytes, half v_sub % 2 of chunk v_sub / 2)
                u32x2 *vs = (u32x2 *)&vst[wave][0];
#pragma unroll
                for (int p = 0; p < VP; ++p) {
                    const int k = p * VKP + v_key;
                    vs[(k * CH + ((v_sub >> 1) ^ (k & (CH - 1)))) * 2 + (v_sub & 1)] = vt[p];
                }
            }
#pragma unroll
            for (int g16 = 0; g16 < NG; ++g16) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int k = g16 * 16 + qrow;
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const u32x4 w = kst[wave][k * CH + ((qgrp + 4 * (m >> 1)) ^ (k & (CH - 1)))];
                    const int i = 2 * (m & 1);
                    u32x4 kv;
                    kv[0] = H::template from_e4m3<false>(w[i]);
                    kv[1] = H::template from_e4m3<true>(w[i]);
                    kv[2] = H::template from_e4m3<false>(w[i + 1]);
                    kv[3] = H::template from_e4m3<true>(w[i + 1]);
                    const u32x4 qv = {qr[m][0], qr[m][1], qr[m][2], qr[m][3]};
                    acc = H::mma(qv, kv, acc);
                }
                const int j = t0 + g16 * 16 + qrow;
                const bool ok = j >= jlo && j < jhi;
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    float v = acc[g] * k_scale;
                    if constexpr (ALIBI) v = __builtin_fmaf((float)(L - 1 - j), alibi_raw[g], v);
                    s[g16][g] = ok ? v : -INFINITY;
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < SP; ++p) {
                const int j = t0 + p * SKP + s_key;
                const bool ok = j >= jlo && j < jhi;
                // this lane's 16 dims of the key as 8 bf16 pairs, in qr's order
                unsigned kw[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kw[i] = kt[p][0][i];
                    kw[4 + i] = kt[p][1][i];
                }
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = H::dot(kw[i], qr[g][i], acc);
                    acc = group_sum<SL>(acc);
                    if constexpr (ALIBI) acc = __builtin_fmaf((float)(L - 1 - j), alibi_raw[g], acc);
                    s[p][g] = ok ? acc : -INFINITY;
                }
            }
        }
        // tile max per head over the wavefront, then the lazy reference update
        bool move = false;
        float m_new[GT];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float mt = s[0][g];
#pragma unroll
            for (int p = 1; p < KA; ++p) mt = fmaxf(mt, s[p][g]);
            // (matrix path: lane 0's row holds the keys; the other rows' values are not read)
            mt = QKM ? row_max16(mt) : across_groups_max<SL>(mt);
            mt = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mt)));
            m_new[g] = fmaxf(m_ref[g], mt * c2);
            move |= m_new[g] > m_ref[g] + RESCALE_THRESHOLD;
        }
        if (move) {                                  // uniform across the wavefront
            float alpha_my = 1.f, alpha_q = 1.f;
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const bool mv = m_new[g] > m_ref[g] + RESCALE_THRESHOLD;
                const float alpha = mv ? __builtin_amdgcn_exp2f(m_ref[g] - m_new[g]) : 1.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[g][e] *= alpha;
                l_acc[g] *= alpha;
                if (g == my_g) alpha_my = alpha;
                alpha_q = (qrow == g) ? alpha : alpha_q;
                if (mv) m_ref[g] = m_new[g];
            }
            l_part *= alpha_my;
            if constexpr (PVM) {
#pragma unroll
                for (int mm = 0; mm < ND; ++mm)
#pragma unroll
                    for (int e = 0; e < 4; ++e) ot[mm][e] *= alpha_q;
            }
        }
        // P of head my_g for this lane's keys, into the wavefront's LDS slot
        // (the reads go through readfirstlane, which the values allow: as plain
        // reads of m_ref the compiler turns this choice into one indexed read
        // and moves m_ref out of registers into LDS)
        auto uni = [](float x) __attribute__((always_inline)) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
        };
        if constexpr (QKM) {
            // lanes 0-15: P of every head for key l % 16 of each group
            float m_use[GT];
#pragma unroll
            for (int g = 0; g < GT; ++g) m_use[g] = (m_ref[g] == -INFINITY) ? 0.f : m_ref[g];
            if (lane < 16) {
#pragma unroll
                for (int g16 = 0; g16 < NG; ++g16) {
                    float pv[GT];
#pragma unroll
                    for (int g = 0; g < GT; ++g) {
                        pv[g] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[g16][g], c2, -m_use[g]));
                        l_acc[g] += pv[g];
                    }
                    if constexpr (PVM) {
#pragma unroll
                        for (int g = 0; g < GT; ++g) pwt[wave][g][g16 * 16 + qrow] = pv[g];
                    } else {
                        float *dst = &pw[wave][g16 * 16 + qrow][0];
                        if constexpr (GT == 4) *(float4 *)dst = make_float4(pv[0], pv[1], pv[2], pv[3]);
                        else if constexpr (GT == 2) *(float2 *)dst = make_float2(pv[0], pv[1]);
                        else dst[0] = pv[0];
                    }
                }
            }
        } else {
            float m_my = uni(m_ref[0]);
#pragma unroll
            for (int g = 1; g < GT; ++g) m_my = (my_g == g) ? uni(m_ref[g]) : m_my;
            const float m_use = (m_my == -INFINITY) ? 0.f : m_my;
#pragma unroll
            for (int p = 0; p < SP; ++p) {
                float sv = s[p][0];
#pragma unroll
                for (int g = 1; g < GT; ++g) sv = (my_g == g) ? s[p][g] : sv;
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c2, -m_use));
                if (s_sub < GT) {
                    l_part += pv;
                    pw[wave][p * SKP + s_key][s_sub] = pv;
                }
            }
        }
        // P.V in the value layout, two keys at a time: a lane holds the same 8
        // dims of keys p and p+1 (passes p, p+1); v_perm_b32 pairs their values
        // per dim and v_dot2_f32_bf16 multiplies them with the pair of P values
        // (bf16, as for the matrix product of the prefill; fp32 accumulate)
        static_assert(VP % 2 == 0, "value passes come in pairs");
        if constexpr (PVM) {
            // P^T operand: keys 8 qgrp .. +8 of head qrow (zero past the heads)
            const int hq = qrow < GT ? qrow : 0;
            const float4 x = *(const float4 *)&pwt[wave][hq][8 * qgrp];
            const float4 y = *(const float4 *)&pwt[wave][hq][8 * qgrp + 4];
            u32x4 pb = {H::pack(x.x, x.y), H::pack(x.z, x.w), H::pack(y.x, y.y), H::pack(y.z, y.w)};
            if (qrow >= GT) pb = u32x4{0u, 0u, 0u, 0u};
            const char *vs = (const char *)&vst[wave][0];
            const int row = 8 * qgrp + (qrow >> 1);
#pragma unroll
            for (int mm = 0; mm < ND; ++mm) {
                const int off = row * D + ((mm ^ (row & (CH - 1))) << 4) + 8 * (qrow & 1);
                const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2 *)(vs + off));
                u32x4 va;
                va[0] = H::template from_e4m3<false>((unsigned)w[0]);
                va[1] = H::template from_e4m3<true>((unsigned)w[0]);
                va[2] = H::template from_e4m3<false>((unsigned)w[1]);
                va[3] = H::template from_e4m3<true>((unsigned)w[1]);
                ot[mm] = H::mma(va, pb, ot[mm]);
            }
        } else {
#pragma unroll
        for (int p = 0; p < VP; p += 2) {
            float pa[GT], pb[GT];
            const float *src0 = &pw[wave][p * VKP + v_key][0];
            const float *src1 = &pw[wave][(p + 1) * VKP + v_key][0];
            if constexpr (GT == 4) {
                const float4 x = *(const float4 *)src0, y = *(const float4 *)src1;
                pa[0] = x.x; pa[1] = x.y; pa[2] = x.z; pa[3] = x.w;
                pb[0] = y.x; pb[1] = y.y; pb[2] = y.z; pb[3] = y.w;
            } else if constexpr (GT == 2) {
                const float2 x = *(const float2 *)src0, y = *(const float2 *)src1;
                pa[0] = x.x; pa[1] = x.y;
                pb[0] = y.x; pb[1] = y.y;
            } else {
                pa[0] = src0[0];
                pb[0] = src1[0];
            }
            unsigned pp[GT];
#pragma unroll
            for (int g = 0; g < GT; ++g) pp[g] = H::pack(pa[g], pb[g]);
            // this lane's 8 dims of keys p and p + 1 as bf16 pairs
            unsigned wa[4], wb[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if constexpr (KV8) {
                    wa[2 * i] = H::template from_e4m3<false>(vt[p][i]);
                    wa[2 * i + 1] = H::template from_e4m3<true>(vt[p][i]);
                    wb[2 * i] = H::template from_e4m3<false>(vt[p + 1][i]);
                    wb[2 * i + 1] = H::template from_e4m3<true>(vt[p + 1][i]);
                } else {
                    wa[2 * i] = vt[p][2 * i];
                    wa[2 * i + 1] = vt[p][2 * i + 1];
                    wb[2 * i] = vt[p + 1][2 * i];
                    wb[2 * i + 1] = vt[p + 1][2 * i + 1];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned va = wa[i], vb = wb[i];                           // dims 2i, 2i+1
                const unsigned even = __builtin_amdgcn_perm(vb, va, 0x05040100u);  // (va.lo, vb.lo)
                const unsigned odd = __builtin_amdgcn_perm(vb, va, 0x07060302u);   // (va.hi, vb.hi)
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    o[g][2 * i] = H::dot(pp[g], even, o[g][2 * i]);
                    o[g][2 * i + 1] = H::dot(pp[g], odd, o[g][2 * i + 1]);
                }
            }
        }
        }
    };

    // ---- tile loop: NBUF-1 tiles' loads are in flight during each compute ---
    // Loads are issued on every path, also for tiles past tb (their keys all
    // clamp to row jhi-1: one cached row, no HBM traffic), and tiles go in
    // groups of NBUF (a tile past tb has every key masked: p = 0 against
    // finite rows), so each loop iteration is the same load/compute sequence
    // and the compiler waits only for the tile in use.
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) load(ta + i, kb[i], vb[i]);
    for (int t = ta; t < tb; t += NBUF) {
#pragma unroll
        for (int i = 0; i < NBUF; ++i) {
            load(t + i + NBUF - 1, kb[(i + NBUF - 1) % NBUF], vb[(i + NBUF - 1) % NBUF]);
            compute(t + i, kb[i], vb[i]);
        }
    }

    // ---- merge: lanes of a wavefront, then the four wavefronts ------------
    // P.V: lanes with the same dims (v_sub) hold different keys
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[g][e];
            if constexpr (VL == 8) x += xor8(x);
            x += xor16(x);
            x += xor32(x);
            o[g][e] = x;
        }
    // row sum of head my_g: lanes with the same s_sub hold different keys
    // (matrix path: every head's sum, over the lanes of row 0)
    const float lsum = QKM ? 0.f : across_groups_sum<SL>(l_part);
    float lsum_g[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) lsum_g[g] = QKM ? row_sum16(l_acc[g]) : 0.f;
    if constexpr (PVM) {
        // O^T: lane l holds dims 16 mm + 4 qgrp .. +4 of head qrow
        if (qrow < GT) {
#pragma unroll
            for (int mm = 0; mm < ND; ++mm)
                *(float4 *)&mo[wave][qrow][16 * mm + 4 * qgrp] = make_float4(ot[mm][0], ot[mm][1], ot[mm][2], ot[mm][3]);
        }
    } else if (v_key == 0) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            *(float4 *)&mo[wave][g][v_sub * 8] = make_float4(o[g][0], o[g][1], o[g][2], o[g][3]);
            *(float4 *)&mo[wave][g][v_sub * 8 + 4] = make_float4(o[g][4], o[g][5], o[g][6], o[g][7]);
        }
    }
    if constexpr (QKM) {
        if (lane == 0) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                mml[wave][g][0] = m_ref[g];
                mml[wave][g][1] = lsum_g[g];
            }
        }
    } else if (s_key == 0 && s_sub < GT) {
        mml[wave][s_sub][0] = m_ref[0];
#pragma unroll
        for (int g = 1; g < GT; ++g)
            if (s_sub == g) mml[wave][s_sub][0] = m_ref[g];
        mml[wave][s_sub][1] = lsum;
    }
    __syncthreads();
    for (int idx = tid; idx < GT * D; idx += NTHREADS) {
        const int g = idx / D, d = idx - (idx / D) * D;
        float M = mml[0][g][0];
#pragma unroll
        for (int w = 1; w < NWAVES; ++w) M = fmaxf(M, mml[w][g][0]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float acc = 0.f, lacc = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            const float wt = __builtin_amdgcn_exp2f(mml[w][g][0] - M_use);
            acc = __builtin_fmaf(wt, mo[w][g][d], acc);
            lacc = __builtin_fmaf(wt, mml[w][g][1], lacc);
        }
        const int64_t row = ((int64_t)b * a.heads_q + h0 + g) * a.max_chunks + chunk;
        a.ws_o[row * D + d] = KV8 ? acc * v_scale : acc;
        if (d == 0) {
            a.ws_ml[row * 2 + 0] = M;
            a.ws_ml[row * 2 + 1] = lacc;
        }
    }
}

template <int D, int GT, bool ALIBI, bool PAGED, bool KV8, int KT, bool F16>
__global__ __launch_bounds__(NTHREADS) void decode_split_kernel(DecodeArgs a) {
    decode_split<D, GT, ALIBI, PAGED, KV8, KT, F16>(a);
}

// The FP8 cache's matrix-core accumulators would otherwise go to extra
// accumulation registers, leaving two wavefronts per SIMD; asking for three
// keeps them in the ordinary ones.
template <int D, int GT, bool ALIBI, bool PAGED, int KT, bool F16>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(3))) void decode_split_fp8_kernel(DecodeArgs a) {
    decode_split<D, GT, ALIBI, PAGED, true, KT, F16>(a);
}

// Item table of a batch of more than 64 sequences, written once per call
// (one workgroup): items[0] = number of items, items[1 + i] = b * max_chunks
// + chunk of item i, in the order rank_block defines.  Sixteen wavefronts
// rank sixteen blocks at a time; a running base carries the items of the
// blocks before them.
constexpr int PLAN_THREADS = 1024;

__global__ __launch_bounds__(PLAN_THREADS) void decode_plan_kernel(DecodeArgs a) {
    constexpr int NW = PLAN_THREADS / 64;
    __shared__ int block_total[NW];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int base = 0;
    for (int r0 = 0; r0 < a.batch; r0 += NW * 64) {
        const int b0 = r0 + wave * 64;
        int n = 0, ahead = 0, total = 0, L_lane;
        if (b0 < a.batch) rank_block(a, b0, lane, n, ahead, total, L_lane);
        if (lane == 0) block_total[wave] = total;
        __syncthreads();
        int excl = base, round_total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            excl += (w < wave) ? block_total[w] : 0;
            round_total += block_total[w];
        }
        for (int c = 0; c < n; ++c) a.ws_items[1 + excl + ahead + c] = (b0 + lane) * a.max_chunks + c;
        base += round_total;
        __syncthreads();                           // block_total is rewritten next round
    }
    if (threadIdx.x == 0) a.ws_items[0] = base;
}

// One wavefront per (sequence, query head), four per workgroup.  The partial
// P.V rows of the first 8 chunks are loaded before anything else, together
// with every chunk's (m, l), so a sequence with at most 8 chunks (the usual
// case: the library picks chunks of up to 2048 keys) costs one memory round
// trip; longer ones loop over further groups of 8.  Each lane owns D / 64
// dims of O.
constexpr int COMBINE_THREADS = 256;
constexpr int COMBINE_GROUP = 8;     // partial rows loaded per round trip

template <int D, bool F16>
__global__ __launch_bounds__(COMBINE_THREADS) void decode_combine_kernel(DecodeArgs a) {
    constexpr int DPL = D / 64;              // dims per lane
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * (COMBINE_THREADS / 64) + (threadIdx.x >> 6);
    if (bh >= a.batch * a.heads_q) return;
    const int b = bh / a.heads_q, h = bh - (bh / a.heads_q) * a.heads_q;
    int lo, L, n, len;
    visible_range(a, b, lo, L);
    chunking(a, lo, L, n, len);
    (void)len;
    const int64_t base = ((int64_t)b * a.heads_q + h) * a.max_chunks;
    const float *wo = a.ws_o + base * D + lane * DPL;
    const float *wml = a.ws_ml + base * 2;

    float ov[COMBINE_GROUP][DPL];
#pragma unroll
    for (int u = 0; u < COMBINE_GROUP; ++u)
#pragma unroll
        for (int i = 0; i < DPL; ++i) ov[u][i] = u < n ? wo[(int64_t)u * D + i] : 0.f;
    float M = -INFINITY;
    for (int j = lane; j < n; j += 64) M = fmaxf(M, wml[2 * j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float M_use = (M == -INFINITY) ? 0.f : M;

    float acc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
    float Lsum = 0.f;                        // the same in every lane
    for (int j0 = 0; j0 < n; j0 += COMBINE_GROUP) {
        if (j0 > 0) {
#pragma unroll
            for (int u = 0; u < COMBINE_GROUP; ++u)
#pragma unroll
                for (int i = 0; i < DPL; ++i) ov[u][i] = j0 + u < n ? wo[(int64_t)(j0 + u) * D + i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < COMBINE_GROUP; ++u) {
            if (j0 + u < n) {
                const float w = __builtin_amdgcn_exp2f(wml[2 * (j0 + u)] - M_use);
                Lsum = __builtin_fmaf(w, wml[2 * (j0 + u) + 1], Lsum);
#pragma unroll
                for (int i = 0; i < DPL; ++i) acc[i] = __builtin_fmaf(w, ov[u][i], acc[i]);
            }
        }
    }

    const bool ok = Lsum > 0.f;
    const float inv = ok ? 1.f / Lsum : 0.f;
    unsigned short *orow = (unsigned short *)a.o + b * a.o_sb + h * a.o_sh + lane * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
        const typename H16<F16>::t x = (typename H16<F16>::t)(acc[i] * inv);
        orow[i] = __builtin_bit_cast(unsigned short, x);
    }
    if (a.lse && lane == 0)
        a.lse[(int64_t)b * a.heads_q + h] = ok ? (M_use + log2f(Lsum)) * LN2 : -INFINITY;
}

// Tile length: 16 keys, or 32 for an FP8 cache (the same bytes per tile as
// bf16, so as many bytes in flight per wavefront) when pages allow it.
int tile_keys(const DecodeArgs &a) {
    return (a.kv_fp8 && (!a.block_table || a.page_size % 32 == 0)) ? 32 : 16;
}

template <int D, bool F16, int GT, bool ALIBI, bool PAGED>
void launch_split_kv(const DecodeArgs &a, dim3 grid, hipStream_t s) {
    if (!a.kv_fp8)
        hipLaunchKernelGGL((decode_split_kernel<D, GT, ALIBI, PAGED, false, 16, F16>), grid, dim3(NTHREADS), 0, s, a);
    else if (tile_keys(a) == 32)
        hipLaunchKernelGGL((decode_split_fp8_kernel<D, GT, ALIBI, PAGED, 32, F16>), grid, dim3(NTHREADS), 0, s, a);
    else
        hipLaunchKernelGGL((decode_split_fp8_kernel<D, GT, ALIBI, PAGED, 16, F16>), grid, dim3(NTHREADS), 0, s, a);
}

template <int D, bool F16, int GT, bool ALIBI>
void launch_split_paged(const DecodeArgs &a, dim3 grid, hipStream_t s) {
    if (a.block_table) launch_split_kv<D, F16, GT, ALIBI, true>(a, grid, s);
    else launch_split_kv<D, F16, GT, ALIBI, false>(a, grid, s);
}

template <int D, bool F16, int GT>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)(a.heads_kv * a.head_groups) * a.batch * a.max_chunks);
    if (a.alibi) launch_split_paged<D, F16, GT, true>(a, grid, s);
    else launch_split_paged<D, F16, GT, false>(a, grid, s);
    return hipGetLastError();
}

template <int D, bool F16>
hipError_t launch_all(const DecodeArgs &a, int gt, hipStream_t s) {
    hipError_t e;
    if (a.ws_items) {
        hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    switch (gt) {
        case 1: e = launch_split<D, F16, 1>(a, s); break;
        case 2: e = launch_split<D, F16, 2>(a, s); break;
        default: e = launch_split<D, F16, 4>(a, s); break;
    }
    if (e != hipSuccess) return e;
    const int per_wg = COMBINE_THREADS / 64;
    hipLaunchKernelGGL((decode_combine_kernel<D, F16>), dim3((a.batch * a.heads_q + per_wg - 1) / per_wg),
                       dim3(COMBINE_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &args, int head_dim, int heads_per_wg, bool f16,
                              hipStream_t s) {
    DecodeArgs a = args;
    a.origin_align = a.block_table ? tile_keys(a) : 1;
    if (f16) {
        if (head_dim == 128) return launch_all<128, true>(a, heads_per_wg, s);
        return launch_all<64, true>(a, heads_per_wg, s);
    }
    if (head_dim == 128) return launch_all<128, false>(a, heads_per_wg, s);
    return launch_all<64, false>(a, heads_per_wg, s);
}

}  // namespace fa
