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
// Work decomposition: one workgroup = 8 wavefronts of 32 query rows each,
// over one (batch, KV head): 256 / GP positions of GP query heads that share
// that KV head (GP = gcd(heads_q / heads_kv, 8): 1 for MHA), so every K/V
// tile in LDS serves GP heads and, under a window, the workgroup's key span
// covers fewer positions.  Wavefront w takes head w % GP and positions
// 32 (w / GP) .. + 31 of the workgroup's.
//   * grid = query tiles x (batch, KV head, head slice); heads and batches
//     are independent work items spread over all CUs (jsqmd.com page, section
//     二 "multi-head parallel strategy").  Consecutive workgroup ids differ in
//     (batch, KV head) first, so the dispatcher's round-robin over the 8 XCDs
//     keeps each KV head's K/V inside one XCD's L2; under a causal mask the
//     longest query tiles are dispatched first.
//   * KV tiles of 64 keys move HBM -> LDS with direct-to-LDS loads
//     (global_load_lds_dwordx4: no VGPR staging) into two K and two V buffers
//     shared by all 8 wavefronts: the next tiles stream in while the current
//     ones are read (the two-region ping-pong of the hwcomputing.csdn.net
//     page, section 2.1).
//   * the causal / window / valid-length masks are index arithmetic: tiles
//     wholly outside a wavefront's visible band are skipped by that
//     wavefront, and the element mask runs only on tiles that cross a
//     boundary (jsqmd.com page, section 二 "causal mask and decode").  Rows
//     at or beyond the valid key length are never read: their loads are
//     redirected to the last valid row and their scores masked
//     (agent.csdn.net BERT page, chapter 四).
//
// Matrix/vector overlap (the page's Cube/Vector pipelining, jsqmd.com
// section 二, done the gfx950 way): the 8 wavefronts form two groups of 4,
// one wavefront of each group per SIMD.  Time is cut into phases, two per
// tile, with a workgroup barrier after every second one; in every phase one
// group runs its matrix step (PV of the previous tile, then S = K Q^T of the
// current tile: 32 MFMAs) while the other group runs its softmax step on the
// VALU (max, exp, P in bf16, row sums, rare O rescale).  Group B lags group
// A by one phase, so each SIMD has one wavefront feeding the matrix core and
// one feeding the vector ALU.
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
// Softmax bookkeeping: P is taken against a per-row reference, not the exact
// running max.  A tile first computes P against the current reference; only
// when some row has no reference yet, or a lane's P sum for the tile passes
// 2^16 (so no P can have passed it), does the wavefront compute the exact row
// max and move the reference of the rows whose max passed it by more than 8
// in the base-2 exponent domain (a factor 2^8), rescale O and the row sum,
// and recompute P.  O, the row sum and P always share one reference, so the
// result is exact up to rounding; the row max and the rescale work are
// skipped on almost every tile.  The row sum adds the fp32 P values (before
// their bf16 rounding for the PV product), so LSE carries only fp32 rounding.
#include "fa_internal.h"

#include <climits>
#include <cmath>

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;

constexpr int BM = kPrefillBM;   // query rows per workgroup
constexpr int BN = 64;           // keys per KV tile
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
static_assert(BM == NWAVES * 32, "one 32-row block per wavefront");
constexpr float LN2 = 0.693147180559945309f;
constexpr float RESCALE_THRESHOLD = 8.0f;   // log2 of the largest un-rescaled p
// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int SG_MFMA = 0x008;
constexpr int SG_DS_READ = 0x100;

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
    static constexpr int LOADS_PER_WAVE = BYTES / 1024 / NWAVES;
    // physical chunk of logical chunk c in row r
    __host__ __device__ static constexpr int k_chunk(int r, int c) { return c ^ ((r / RPW) & (CH - 1)); }
    __host__ __device__ static constexpr int v_chunk(int r, int c) {
        return c ^ ((((r / RPW) & 3) << 2) & (CH - 1));
    }
};

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, r);
}

// The 16-bit element type of Q, K, V, O (and of P in the P.V product):
// bf16, or IEEE half with F16.  Both use the same 32x32x16 MFMA shape with
// fp32 accumulation and the same operand layouts.
template <bool F16> struct E16;
template <> struct E16<false> {
    using t = __bf16;
    using v8 = bf16x8;
    // fast-path bound on a lane's P sum (keeps every P far inside the type)
    // fast-path bound on the P values of one lane's share of a tile: 2^16
    // keeps bf16 P and the fp32 accumulators far from overflow
    static constexpr float FAST_BOUND = 65536.0f;
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack(float lo, float hi) { return pack_bf16x2(lo, hi); }
    static __device__ __forceinline__ float lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
    static __device__ __forceinline__ float hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
    static __device__ __forceinline__ float one(unsigned short b) {
        return __builtin_bit_cast(float, (unsigned)b << 16);
    }
    // the largest bf16 value at or below x >= 0 (the upper 16 bits)
    static __device__ __forceinline__ t down(float x) {
        return __builtin_bit_cast(t, (unsigned short)(__builtin_bit_cast(unsigned, x) >> 16));
    }
};
template <> struct E16<true> {
    using t = _Float16;
    using v8 = f16x8;
    // half tops out at 65504: P sums stay at or below 2^14
    static constexpr float FAST_BOUND = 16384.0f;
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack(float lo, float hi) {
        f16x2 r;
        r[0] = (_Float16)lo;
        r[1] = (_Float16)hi;
        return __builtin_bit_cast(unsigned, r);
    }
    static __device__ __forceinline__ float lo(unsigned w) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(unsigned w) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
    }
    static __device__ __forceinline__ float one(unsigned short b) {
        return (float)__builtin_bit_cast(_Float16, b);
    }
    // the largest half value at or below x >= 0 (nearest, stepped down one
    // unit when it rounded up; half bit patterns of x >= 0 are ordered)
    static __device__ __forceinline__ t down(float x) {
        const _Float16 h = (_Float16)x;
        return (float)h > x ? __builtin_bit_cast(_Float16, (unsigned short)(__builtin_bit_cast(unsigned short, h) - 1))
                            : h;
    }
};

// Workgroup barrier of the phase loop.  __syncthreads() would also drain
// every outstanding vector-memory operation of the wavefront (its fence is
// lowered with vmcnt(0)), i.e. wait for the direct-to-LDS loads issued at the
// start of the phase, which no reader needs before the next odd phase; this
// barrier only drains the wavefront's LDS reads.  Where the loads must have
// landed, wait_loads() comes first.  The memory clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void phase_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_loads() {
    // vmcnt(0); expcnt and lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Combine a value with the one held by the partner lane (lane ^ 32) using
// v_permlane32_swap, a VALU lane swap, instead of a ds_bpermute shuffle that
// would queue in the LDS pipe behind the matrix wavefront's operand reads.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// One direct-to-LDS load: each lane moves 16 bytes from its global address g
// to LDS address la + 16 * lane, la being the wavefront-uniform 32-bit LDS
// address of lane 0 (passed in M0, which needs one wait state before the load
// reads it).  Issued as inline assembly so that the compiler's wait-count pass
// does not see an in-flight load that also writes LDS: it would then drain
// every LDS read of the loop to zero (lgkmcnt(0)) while the load is
// outstanding.  Completion is tracked explicitly with wait_loads() and the
// barrier after it.  The LDS address travels as a 32-bit LDS offset: from a
// generic pointer the compiler would read it back with two readfirstlanes and
// a null check per load, on the critical softmax step of the lagging group.
__device__ __forceinline__ void lds_dma16(const char *g, unsigned la) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(la))
                 : "memory", "m0");
}

// 32-bit LDS address of a location in a __shared__ array
__device__ __forceinline__ unsigned lds_addr(const char *l) {
    return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char *)l;
}

// The same load with a wavefront-uniform base address (in SGPRs) and a 32-bit
// per-lane offset, which holds one VGPR per load instead of two.
__device__ __forceinline__ void lds_dma16_s(const char *base, unsigned off, unsigned la) {
    // the base is the same in every lane; readfirstlane makes that visible,
    // so that it lives in SGPRs as the instruction's base operand requires
    const uint64_t bu = (uint64_t)(uintptr_t)base;
    base = (const char *)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((unsigned)(bu >> 32)) << 32) |
                                     (unsigned)__builtin_amdgcn_readfirstlane((unsigned)bu));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(la))
                 : "memory", "m0");
}

// D: head_dim; ALIBI: add the per-head linear bias -m |pos - j| to the scores;
// ROPE: rotate the query rows (RoPE) as they are loaded (keys arrive rotated);
// MASK: add an explicit additive mask read from memory (1: any mask, added in
// the softmax step; 2: a key mask, the same row for every query, added by the
// matrix cores as one more k-step of the S product); F16: the inputs are
// IEEE half instead of bf16; PACK: a.gqa_pack query heads share the
// workgroup (without it one head, and the work-item arithmetic is constant);
// PERSIST (with PACK, no biases): one workgroup per CU walks the work items
// (see below) instead of one workgroup per item.
template <int D, bool ALIBI, bool ROPE, int MASK, bool F16, bool PACK, bool PERSIST>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2)))
void prefill_bf16_kernel(PrefillArgs a) {
    static_assert(!PERSIST || (PACK && !ALIBI && !ROPE && MASK == 0 && D == 128), "persistent form: packed, no biases");
    static_assert(MASK >= 0 && MASK <= 2, "mask kind");
    using T = Tile<D>;
    using E = E16<F16>;
    using v8 = typename E::v8;
    using et = typename E::t;
    constexpr int KSTEPS = D / 16;        // MFMA k-steps over head_dim for S
    constexpr int DBLK = D / 32;          // 32-dim row blocks of O^T

    __shared__ __attribute__((aligned(1024))) char sK0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char sK1[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char sV0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char sV1[T::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave >> 2;            // 0: leading group, 1: lagging group
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // ---- work item --------------------------------------------------------
    const int GP = PACK ? a.gqa_pack : 1;             // query heads per workgroup
    auto locate = [&](unsigned wi, int &rank, int &b, int &h, int &kvh) __attribute__((always_inline)) {
        if constexpr (PACK) {
            const int slices = a.group / GP;          // workgroups per (position block, KV head)
            const int units = a.batch * a.heads_kv * slices;
            rank = wi / units;
            const int unit = wi - rank * units;
            b = unit / (a.heads_kv * slices);
            const int kvh_slice = unit - b * (a.heads_kv * slices);
            kvh = kvh_slice / slices;
            // this wavefront's query head (uniform across it)
            h = __builtin_amdgcn_readfirstlane(kvh * a.group + (kvh_slice - kvh * slices) * GP + wave % GP);
        } else {
            const int bh_count = a.batch * a.heads_q;
            rank = wi / bh_count;
            const int bh = wi - rank * bh_count;
            b = bh / a.heads_q;
            h = bh - b * a.heads_q;
            kvh = h / a.group;
        }
    };
    // PERSIST: G workgroups (one per CU) take the items in rounds of G, in
    // snake order (round r: workgroup w takes r G + w, or r G + G - 1 - w
    // when r is odd), which keeps the heavy-first order of the items balanced
    // across workgroups.  Once an item's tile loop is done, its LDS tiles are
    // free: each wavefront loads its 32 rows of the next item's Q into 8 KiB
    // of them (direct-to-LDS, 16-byte chunks XOR-swizzled by row) before it
    // writes the current item's O, so the Q load overlaps the O write
    // instead of starting the next item.
    const int n_items = PERSIST ? a.num_q_tiles * (a.heads_q / GP) * a.batch : 0;
    auto item_of = [&](int r) __attribute__((always_inline)) {
        const int G = (int)gridDim.x, w = (int)blockIdx.x;
        return r * G + ((r & 1) ? G - 1 - w : w);
    };
    // wavefront w's Q staging area: half w % 2 of tile buffer w / 2
    auto q_stage = [&]() __attribute__((always_inline)) {
        char *buf = (wave >> 1) == 0 ? sK0 : (wave >> 1) == 1 ? sK1 : (wave >> 1) == 2 ? sV0 : sV1;
        return buf + (wave & 1) * 8192;
    };
    // the tile buffers' LDS addresses, and this wavefront's index as a
    // uniform value (its share of a tile)
    const unsigned lK0 = lds_addr(sK0), lK1 = lds_addr(sK1), lV0 = lds_addr(sV0), lV1 = lds_addr(sV1);
    const unsigned wave_u = (unsigned)__builtin_amdgcn_readfirstlane(wave);
    bool have_next = false;
    for (int round = 0;; ++round) {
    const unsigned wi = PERSIST ? (unsigned)item_of(round) : blockIdx.x;
    if (PERSIST && (int)wi >= n_items) break;
    int rank, b, h, kvh;
    locate(wi, rank, b, h, kvh);
    const int qtile = a.causal ? (a.num_q_tiles - 1 - rank) : rank;

    int Lq = a.seqlen_q, Lk = a.seqlen_k;
    if (a.seqlens_q) Lq = min(max(a.seqlens_q[b], 0), a.seqlen_q);
    if (a.seqlens_k) Lk = min(max(a.seqlens_k[b], 0), a.seqlen_k);
    const int wg_rows = PACK ? BM / GP : BM;   // positions per workgroup
    const int q0 = qtile * wg_rows;
    const int offset = Lk - Lq;           // bottom-right causal alignment
    const int W = a.window_left;
    // RoPE: rows before position 0 (i < Lq - Lk) have no angle in the tables
    // and see no key; the valid rows are [q_first, Lq)
    const int q_first = ROPE ? max(0, -offset) : 0;

    // visible key range [lo, hi) of a block of rows [r0, r1] (all valid)
    auto key_range = [&](int r0, int r1, int &lo, int &hi) {
        lo = 0;
        hi = Lk;
        if (a.causal) hi = min(hi, r1 + offset + 1);
        if (W > 0) lo = max(0, r0 + offset - W + 1);
    };
    int wg_lo = 0, wg_hi = 0;
    const int wg_r0 = ROPE ? max(q0, q_first) : q0;
    if (wg_r0 < min(q0 + wg_rows, Lq)) key_range(wg_r0, min(q0 + wg_rows, Lq) - 1, wg_lo, wg_hi);
    const int t_begin = wg_lo / BN;
    const int ntiles = (wg_hi > wg_lo) ? (wg_hi + BN - 1) / BN - t_begin : 0;

    const int q0w = q0 + (PACK ? wave / GP : wave) * 32;   // first query row of this wavefront
    const int qi = q0w + l32;             // this lane's query row
    // tiles (relative to t_begin) this wavefront has to visit: [w_lo, w_hi)
    int w_lo = 0, w_hi = 0;
    const int w_r0 = ROPE ? max(q0w, q_first) : q0w;
    if (w_r0 < min(q0w + 32, Lq) && ntiles > 0) {
        int lo, hi;
        key_range(w_r0, min(q0w + 32, Lq) - 1, lo, hi);
        if (hi > lo) {
            w_lo = lo / BN - t_begin;
            w_hi = (hi + BN - 1) / BN - t_begin;
        }
    }

    // Order of the key tiles.  With ALiBi the bias grows toward a row's
    // diagonal, so in key order every tile would raise the row max past the
    // running reference and send the softmax step down its slow exact-max
    // path; visiting the tiles from the last to the first puts the largest
    // scores first.  Step j of the pipeline handles tile tile_of(j); the
    // wavefront's range [w_lo, w_hi) is turned into step numbers to match.
    auto tile_of = [&](int j) { return ALIBI ? ntiles - 1 - j : j; };
    if constexpr (ALIBI) {
        const int lo_ = w_lo;
        w_lo = ntiles - w_hi;
        w_hi = ntiles - lo_;
    }

    const unsigned short *Qp = (const unsigned short *)a.q + b * a.q_sb + h * a.q_sh;
    const char *Kp = (const char *)((const unsigned short *)a.k + b * a.k_sb + kvh * a.k_sh);
    const char *Vp = (const char *)((const unsigned short *)a.v + b * a.v_sb + kvh * a.v_sh);
    const int64_t k_row_bytes = a.k_ss * 2, v_row_bytes = a.v_ss * 2;

    // ---- Q fragment (B operand), zero for rows outside the valid length ---
    v8 qf[KSTEPS];
    bool q_rot = false;                   // RoPE: this lane's row is loaded and gets turned
    if (PERSIST && have_next) {
        // staged by the previous item; then every wavefront has its Q before
        // the first K tile goes into the same buffers
        wait_loads();
        const bool ok = qi < Lq;
        const char *stage = q_stage();
        // (lane indices through an empty asm: the per-lane offsets are then
        // computed here, not hoisted out of the item loop into registers that
        // would stay live across every tile loop)
        int r = l32, hf = half;
        asm volatile("" : "+v"(r), "+v"(hf));
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 v = *(const u32x4 *)(stage + r * 256 + (((2 * ks + hf) ^ (r & 15)) << 4));
            if (!ok) v = u32x4{0u, 0u, 0u, 0u};
            qf[ks] = __builtin_bit_cast(v8, v);
        }
        phase_barrier();
    } else {
        const bool ok = qi < Lq && (!ROPE || qi >= q_first);
        const unsigned short *row = Qp + (int64_t)qi * a.q_ss + half * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok) v = *(const u32x4 *)(row + ks * 16);
            qf[ks] = __builtin_bit_cast(v8, v);
        }
        q_rot = ROPE && ok;
    }

    // RoPE: the lane's 8 dims of a k-step are 4 adjacent pairs, turned by the
    // angles of its row's position (qi + Lk - Lq >= 0 for the rows loaded);
    // the result is rounded to bf16, the operand precision.  Every table read
    // of the row is issued together with the first K tile's loads (one memory
    // round trip; k-steps past rotary_dim read the row's last group of 4 pairs
    // and leave their dims unturned).  The leading group turns its rows before
    // the first barrier; the lagging group, whose first matrix step comes one
    // phase later, turns them while the leading group runs that step.
    float4 rope_c[ROPE ? KSTEPS : 1], rope_s[ROPE ? KSTEPS : 1];
    auto rope_tables = [&]() __attribute__((always_inline)) {
        if constexpr (ROPE) {
            if (q_rot) {
                const int rhalf = a.rotary_dim / 2;
                const float *cr = a.rope_cos + (int64_t)(qi + offset) * rhalf;
                const float *sr = a.rope_sin + (int64_t)(qi + offset) * rhalf;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const int pl = min(ks * 8 + half * 4, rhalf - 4);
                    rope_c[ks] = *(const float4 *)(cr + pl);
                    rope_s[ks] = *(const float4 *)(sr + pl);
                }
            }
        }
    };
    auto rotate_q = [&]() __attribute__((always_inline)) {
        if constexpr (ROPE) {
            if (q_rot) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const int p0 = ks * 8 + half * 4;           // first pair of the 8 dims
                    if (2 * p0 < a.rotary_dim) {                 // rotary_dim: whole groups of 4 pairs
                        const float4 c = rope_c[ks], sn = rope_s[ks];
                        const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = (float)qf[ks][2 * e], y = (float)qf[ks][2 * e + 1];
                            qf[ks][2 * e] = (et)__builtin_fmaf(x, cc[e], -y * ss[e]);
                            qf[ks][2 * e + 1] = (et)__builtin_fmaf(x, ss[e], y * cc[e]);
                        }
                    }
                }
            }
        }
    };

    // ---- HBM -> LDS: each wavefront writes LOADS_PER_WAVE x 1 KiB per tile --
    // For load i the lane's tile row and physical chunk are fixed; only the
    // tile base moves, so full tiles use a uniform base plus a per-lane offset.
    int ld_row[T::LOADS_PER_WAVE];
    unsigned k_loff[T::LOADS_PER_WAVE], v_loff[T::LOADS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
        const int lin = (wave * T::LOADS_PER_WAVE + i) * 1024 + lane * 16;
        const int r = lin / T::ROWB;
        const int p = (lin % T::ROWB) >> 4;
        ld_row[i] = r;
        k_loff[i] = (unsigned)(r * k_row_bytes) + (unsigned)(T::k_chunk(r, p) << 4);
        v_loff[i] = (unsigned)(r * v_row_bytes) + (unsigned)(T::v_chunk(r, p) << 4);
    }
    // (lbuf: the tile buffer's LDS address; full tiles take a uniform base
    // in SGPRs plus the lane's 32-bit offset)
    auto issue = [&](const char *base, int64_t row_bytes, const unsigned *loff, int t, unsigned lbuf,
                     bool is_k) {
        const int k0 = (t_begin + tile_of(t)) * BN;
        const char *tb = base + (int64_t)k0 * row_bytes;
        const unsigned lb = lbuf + wave_u * (T::LOADS_PER_WAVE * 1024);
        if (k0 + BN <= Lk) {
#pragma unroll
            for (int i = 0; i < T::LOADS_PER_WAVE; ++i)
                lds_dma16_s(tb, loff[i], lb + i * 1024);
        } else {
            // last tile: rows past the valid length re-read the last valid row
#pragma unroll
            for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
                const int r = ld_row[i];
                const int lin = (wave * T::LOADS_PER_WAVE + i) * 1024 + lane * 16;
                const int p = (lin % T::ROWB) >> 4;
                const int row = min(k0 + r, Lk - 1);
                const int c = is_k ? T::k_chunk(r, p) : T::v_chunk(r, p);
                lds_dma16(base + (int64_t)row * row_bytes + (c << 4), lb + i * 1024);
            }
        }
    };
    auto issue_k = [&](int t, unsigned lbuf) { issue(Kp, k_row_bytes, k_loff, t, lbuf, true); };
    auto issue_v = [&](int t, unsigned lbuf) { issue(Vp, v_row_bytes, v_loff, t, lbuf, false); };

    // ---- per-lane LDS operand offsets (loop invariant) ----------------------
    const int kr = perm32(l32);                      // K row within a 32-key sub-block
    int k_off[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) k_off[ks] = kr * T::ROWB + (T::k_chunk(kr, ks * 2 + half) << 4);
    const int g16 = lane >> 4, r16 = lane & 15;
    const int v_row_lane = 8 * half + (r16 >> 2);    // + 16 * ksp + 4 * tt
    int v_off[DBLK];
#pragma unroll
    for (int jd = 0; jd < DBLK; ++jd) {
        const int c = 4 * jd + 2 * (g16 & 1) + ((r16 & 3) >> 1);
        v_off[jd] = v_row_lane * T::ROWB + (T::v_chunk(v_row_lane, c) << 4) + (r16 & 1) * 8;
    }

    // ---- per-lane softmax state ----------------------------------------------
    f32x16 oacc[DBLK];
#pragma unroll
    for (int jd = 0; jd < DBLK; ++jd)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[jd][r] = 0.f;
    float m_ref = -INFINITY;   // reference row max, scaled log2 domain
    float l_run = 0.f;         // running row sum over this lane's keys
    f32x16 s[2];               // S^T of the tile in flight (matrix -> softmax step)
    v8 pb[4];                  // P^T of the tile in flight (softmax -> matrix step)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = __builtin_bit_cast(v8, u32x4{0u, 0u, 0u, 0u});

    const int pos = qi + offset;                     // key position of this row
    const float c2 = a.scale_log2;
    const int vis_hi = (ROPE && qi < q_first) ? 0 : (a.causal ? min(Lk, pos + 1) : Lk);
    const int vis_lo = (W > 0) ? pos - W + 1 : INT_MIN;
    // ALiBi in raw score units (the accumulators hold q.k; the exponent is
    // scale_log2 * s): scale * s - m |pos - j| = scale * (s - (m / scale) |pos - j|)
    float alibi_raw = 0.f;
    if constexpr (ALIBI) alibi_raw = -a.alibi[h] / a.scale;
    // explicit mask: this lane's query row (clamped into the tensor for the
    // rows of a partial query tile, whose scores are never used), in raw
    // score units (mask / scale)
    const unsigned short *mrow = nullptr;
    float inv_scale = 0.f;
    if constexpr (MASK == 1) {
        mrow = (const unsigned short *)a.mask + b * a.m_sb + h * a.m_sh +
               (int64_t)min(qi, a.seqlen_q - 1) * a.m_ss;
        inv_scale = 1.f / a.scale;
    }
    // Key mask (MASK == 2): S^T[key][query] gains mask[key] / scale through
    // one more k-step of the S product: the key operand holds the key's mask
    // value m in dims 0-2, the query operand holds 1/scale split into three
    // 16-bit parts (hi and mid rounded down, so that every part is >= 0 and
    // an infinite m never meets parts of both signs; lo rounded to nearest),
    // so the matrix core adds m hi + m mid + m lo: products of 16-bit values
    // are exact in fp32 and the three parts hold all 24 bits of 1/scale, so
    // this is m / scale to fp32 accuracy.  A dim whose part is zero carries 0,
    // not m (an infinite m would give inf * 0).  Lanes of the upper half
    // (dims 8-15) carry zeros.
    v8 qmask = {};
    unsigned kmask_nz = 0;                 // bit 0: mid part nonzero, bit 1: lo part nonzero
    if constexpr (MASK == 2) {
        mrow = (const unsigned short *)a.mask + b * a.m_sb + h * a.m_sh;
        const float inv = 1.f / a.scale;   // > 0 (checked on the host)
        const et ph = E::down(inv);
        const float r1 = inv - (float)ph;
        const et pm = E::down(r1);
        const et pl = (et)(r1 - (float)pm);
        if (half == 0) {
            qmask[0] = ph;
            qmask[1] = pm;
            qmask[2] = pl;
        }
        kmask_nz = ((float)pm != 0.f ? 1u : 0u) | ((float)pl != 0.f ? 2u : 0u);
    }

    // matrix step of tile j: PV of tile j-1 (from vb), then S of tile j (from kb).
    // Operand reads are issued in the order the MFMAs consume them and the
    // schedule keeps the reads a few MFMAs ahead, so LDS latency hides under
    // matrix work instead of stalling every MFMA; consecutive MFMAs use
    // different accumulators.
    // Explicit mask of tile j: loaded at the start of the wavefront's matrix
    // step of tile j, so the loads are in flight during it and have landed
    // by its softmax step (the next step of the same wavefront).  Keys at or
    // beyond seqlen_k are never read.
    u32x4 mpre[2][2];
    auto prefetch_mask = [&](int j) __attribute__((always_inline)) {
        if constexpr (MASK == 1) {
            const int k0 = (t_begin + tile_of(j)) * BN;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int key0 = k0 + sb * 32 + c * 16 + half * 8;
                    if (key0 + 8 <= a.seqlen_k) {
                        mpre[sb][c] = *(const u32x4 *)(mrow + key0);
                    } else {
                        u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (key0 + e < a.seqlen_k)
                                w[e >> 1] |= (unsigned)mrow[key0 + e] << (16 * (e & 1));
                        mpre[sb][c] = w;
                    }
                }
        }
    };
    // Key mask of tile j (MASK == 2): the value of the lane's key row
    // perm32(l32) of each 32-key sub-block, loaded at the end of the
    // wavefront's matrix step of tile j - 1 (before the loop for its first
    // tile); keys at or beyond seqlen_k read nothing and hold 0.
    unsigned kmv[2] = {0u, 0u};
    auto prefetch_kmask = [&](int j) __attribute__((always_inline)) {
        if constexpr (MASK == 2) {
            const int k0 = (t_begin + tile_of(j)) * BN;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const int key = k0 + sb * 32 + kr;
                kmv[sb] = key < a.seqlen_k ? (unsigned)mrow[key] : 0u;
            }
        }
    };
    auto matrix_step = [&](int j, const char *kb, const char *vb) {
        if (j >= w_lo && j < w_hi) prefetch_mask(j);
        if (j - 1 >= w_lo && j - 1 < w_hi) {
            v8 vf[4][DBLK];
#pragma unroll
            for (int ksp = 0; ksp < 4; ++ksp)
#pragma unroll
                for (int jd = 0; jd < DBLK; ++jd) {
                    s16x4 part[2];
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
                        part[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(vb + v_off[jd] +
                                                                        (16 * ksp + 4 * tt) * T::ROWB));
                    vf[ksp][jd] = __builtin_bit_cast(
                        v8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
            for (int ksp = 0; ksp < 4; ++ksp)
#pragma unroll
                for (int jd = 0; jd < DBLK; ++jd)
                    oacc[jd] = E::mfma(vf[ksp][jd], pb[ksp], oacc[jd]);
            // 2 DS reads per MFMA, kept 4 MFMAs ahead
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 8, 0);
#pragma unroll
            for (int i = 0; i < 4 * DBLK - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 4, 0);
        }
        if (j >= w_lo && j < w_hi) {
            v8 kf[KSTEPS][2];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
                    kf[ks][sb] = *(const v8 *)(kb + sb * 32 * T::ROWB + k_off[ks]);
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
            if constexpr (MASK == 2) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const unsigned m = half == 0 ? kmv[sb] : 0u;
                    const unsigned w0 = m | ((kmask_nz & 1u) ? m << 16 : 0u);
                    const unsigned w1 = (kmask_nz & 2u) ? m : 0u;
                    s[sb] = E::mfma(__builtin_bit_cast(v8, u32x4{w0, w1, 0u, 0u}), qmask, s[sb]);
                }
            }
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
                    s[sb] = E::mfma(kf[ks][sb], qf[ks], s[sb]);
            // 1 DS read per MFMA, kept 4 MFMAs ahead (the key-mask products
            // need no read and go first)
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 4, 0);
            if constexpr (MASK == 2) __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
#pragma unroll
            for (int i = 0; i < 2 * KSTEPS - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 4, 0);
            if (j + 1 < w_hi) prefetch_kmask(j + 1);
        }
    };

    // softmax step of tile j: mask, running max, P in bf16, row sums
    auto softmax_step = [&](int j) {
        if (!(j >= w_lo && j < w_hi)) return;
        const int k0 = (t_begin + tile_of(j)) * BN;
        const bool need_mask = (k0 + BN > Lk) ||
                               (a.causal && k0 + BN - 1 > q0w + offset) ||
                               (W > 0 && k0 <= q0w + 31 + offset - W) ||
                               (ROPE && q0w < q_first);
        if constexpr (ALIBI) {
            // distance |pos - key| with key = k0 + half*8 + sb*32 + 16*(r/8) + r%8
            const float base = (float)(pos - k0 - half * 8);
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float dist = fabsf(base - (float)(sb * 32 + ((r >> 3) << 4) + (r & 7)));
                    s[sb][r] = __builtin_fmaf(dist, alibi_raw, s[sb][r]);
                }
        }
        if constexpr (MASK == 1) {
            // the lane's keys are four runs of 8: k0 + 32 sb + 16 c + 8 half + e
            // (prefetched in the matrix step; keys past seqlen_k hold 0)
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned w = mpre[sb][c][e];
                        s[sb][c * 8 + 2 * e] = __builtin_fmaf(E::lo(w), inv_scale, s[sb][c * 8 + 2 * e]);
                        s[sb][c * 8 + 2 * e + 1] = __builtin_fmaf(E::hi(w), inv_scale, s[sb][c * 8 + 2 * e + 1]);
                    }
        }
        if (need_mask) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + sb * 32 + ((r >> 3) << 4) + half * 8 + (r & 7);
                    s[sb][r] = (key >= vis_lo && key < vis_hi) ? s[sb][r] : -INFINITY;
                }
        }
        // P of this tile against the current reference (fast path: no row max)
        auto exps = [&](float m_use, float &psum) __attribute__((always_inline)) {
            psum = 0.f;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    u32x4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][tt * 8 + 2 * i], c2, -m_use));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][tt * 8 + 2 * i + 1], c2, -m_use));
                        w[i] = E::pack(p0, p1);
                        psum += p0 + p1;
                    }
                    pb[sb * 2 + tt] = __builtin_bit_cast(v8, w);
                }
        };
        float psum;
        exps((m_ref == -INFINITY) ? 0.f : m_ref, psum);
        // The fast path stands unless a row has no reference yet, or some P of
        // this lane may exceed FAST_BOUND (its sum does; this also catches an
        // overflow to inf).  Then the wavefront takes the exact row
        // max, moves the reference where it grew past the threshold, rescales
        // O and the row sum, and recomputes P.
        if (__ballot(m_ref == -INFINITY || !(psum <= E::FAST_BOUND))) {
            float mx = s[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
            mx = pair_max(mx);
            const float m_new = fmaxf(m_ref, mx * c2);
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
            exps((m_ref == -INFINITY) ? 0.f : m_ref, psum);
        }
        l_run += psum;
    };

    // ---- phase loop ----------------------------------------------------------
    // Phase p: the leading group runs step p, the lagging group step p - 1;
    // step 2j is the matrix step of tile j, step 2j+1 its softmax step.  At
    // even phase 2j every wavefront issues K of tile j+1 and V of tile j; they
    // must land by the end of phase 2j+1.  Unrolled by four phases so every
    // LDS buffer is named statically.  Only the odd phases end in a barrier:
    // the loads of phase 2j go into the buffers that tile j-1 used, whose
    // last reader (the lagging group's matrix step of tile j-1) ends in phase
    // 2j-1, and tile j+1's buffers are next read in phase 2j+2, after the
    // barrier that follows their wait.  A barrier after the even phases as
    // well, which only kept the two groups in lockstep, measured slightly
    // slower.
    const int nph = ntiles > 0 ? 2 * ntiles + 2 : 0;
    if (ntiles > 0) issue_k(0, lK0);
    if (w_lo < w_hi) prefetch_kmask(w_lo);
    rope_tables();
    if (grp == 0) rotate_q();
    wait_loads();
    __syncthreads();
    if (grp != 0) rotate_q();
    for (int p = 0; p < nph; p += 4) {
        const int j = p >> 1;             // even tile index of this unrolled block
        // phase p (= 2j): leading: matrix(j) ; lagging: softmax(j-1)
        if (j + 1 < ntiles) issue_k(j + 1, lK1);
        if (j < ntiles) issue_v(j, lV0);
        if (grp == 0) matrix_step(j, sK0, sV1);
        else softmax_step(j - 1);
        // phase p+1: leading: softmax(j) ; lagging: matrix(j)
        if (grp == 0) softmax_step(j);
        else matrix_step(j, sK0, sV1);
        wait_loads();
        phase_barrier();
        if (p + 2 >= nph) break;
        // phase p+2 (= 2(j+1)): leading: matrix(j+1) ; lagging: softmax(j)
        if (j + 2 < ntiles) issue_k(j + 2, lK0);
        if (j + 1 < ntiles) issue_v(j + 1, lV1);
        if (grp == 0) matrix_step(j + 1, sK1, sV0);
        else softmax_step(j);
        // phase p+3: leading: softmax(j+1) ; lagging: matrix(j+1)
        if (grp == 0) softmax_step(j + 1);
        else matrix_step(j + 1, sK1, sV0);
        wait_loads();
        phase_barrier();
    }

    // ---- PERSIST: the next item's Q rows into LDS, before O is written ----
    // Every wavefront is past the tile loop's last barrier, so no one reads
    // the tile buffers any more.  Rows past the valid length load a valid
    // row and are zeroed when read.  The load overlaps the O write.
    if constexpr (PERSIST) {
        // (the empty asm hides that nx is the next round's item, so the
        // compiler does not carry this set-up across the next item's loop)
        int nx = item_of(round + 1);
        asm volatile("" : "+s"(nx));
        have_next = nx < n_items;
        if (have_next) {
            int r2, b2, h2, kvh2;
            locate((unsigned)nx, r2, b2, h2, kvh2);
            const int qt2 = a.causal ? (a.num_q_tiles - 1 - r2) : r2;
            int Lq2 = a.seqlen_q;
            if (a.seqlens_q) Lq2 = min(max(a.seqlens_q[b2], 0), a.seqlen_q);
            const int q0w2 = qt2 * wg_rows + (wave / GP) * 32;
            // uniform base at the first row loaded; rows past the valid length
            // clamp to the last valid row (row 0 of an empty sequence)
            const int rb = max(0, min(q0w2, Lq2 - 1));
            const char *qb = (const char *)((const unsigned short *)a.q + b2 * a.q_sb + h2 * a.q_sh +
                                            (int64_t)rb * a.q_ss);
            char *stage = q_stage();
            int ln = lane;                                    // (as above: not hoisted)
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = i * 4 + (ln >> 4);              // row of the 32 this lane's chunk is in
                const int c = (ln & 15) ^ (r & 15);           // the chunk that belongs at this slot
                const int row = max(0, min(q0w2 + r, Lq2 - 1));
                lds_dma16_s(qb, (unsigned)((row - rb) * a.q_ss * 2) + (c << 4), lds_addr(stage + i * 1024));
            }
        }
    }

    // ---- epilogue: normalise once, write O (bf16, RNE) and LSE -------------
    const float l_tot = pair_sum(l_run);
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
                w[0] = E::pack(oacc[jd][4 * j] * inv, oacc[jd][4 * j + 1] * inv);
                w[1] = E::pack(oacc[jd][4 * j + 2] * inv, oacc[jd][4 * j + 3] * inv);
                *(u32x2 *)(orow + d) = w;
            }
        if (a.lse && half == 0) {
            float *lrow = a.lse + ((int64_t)b * a.heads_q + h) * a.seqlen_q;
            lrow[qi] = row_ok ? (m_ref + log2f(l_tot)) * LN2 : -INFINITY;
        }
    }
    if constexpr (!PERSIST) break;
    }   // items
}


template <int D, bool F16, bool ALIBI, bool ROPE>
void launch_mask(const PrefillArgs &a, dim3 grid, dim3 block, hipStream_t s) {
    // GQA packing is built for the bf16 d = 128 kernels; elsewhere one head
    // per workgroup (valid for any group)
    constexpr bool CAN_PACK = D == 128 && !F16;
    constexpr bool CAN_PERSIST = CAN_PACK && !ALIBI && !ROPE;
    // a mask whose rows do not depend on the query (row stride 0) is a key mask
    const int mk = !a.mask ? 0 : (a.m_ss == 0 ? 2 : 1);
    if (a.gqa_pack > 1 && CAN_PERSIST && !a.mask && a.persist_wgs > 0 && grid.x > (unsigned)a.persist_wgs) {
        hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, 0, F16, CAN_PACK, CAN_PERSIST>),
                           dim3(a.persist_wgs), block, 0, s, a);
    } else if (a.gqa_pack > 1 && CAN_PACK) {
        if (mk == 2) hipLaunchKernelGGL((prefill_bf16_kernel<D, ALIBI, ROPE, 2, F16, CAN_PACK, false>), grid, block, 0, s, a);
        else if (mk == 1) hipLaunchKernelGGL((prefill_bf16_kernel<D, ALIBI, ROPE, 1, F16, CAN_PACK, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prefill_bf16_kernel<D, ALIBI, ROPE, 0, F16, CAN_PACK, false>), grid, block, 0, s, a);
    } else {
        if (mk == 2) hipLaunchKernelGGL((prefill_bf16_kernel<D, ALIBI, ROPE, 2, F16, false, false>), grid, block, 0, s, a);
        else if (mk == 1) hipLaunchKernelGGL((prefill_bf16_kernel<D, ALIBI, ROPE, 1, F16, false, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prefill_bf16_kernel<D, ALIBI, ROPE, 0, F16, false, false>), grid, block, 0, s, a);
    }
}

template <int D, bool F16, bool ALIBI>
void launch_rope(const PrefillArgs &a, dim3 grid, dim3 block, hipStream_t s) {
    if (a.rotary_dim > 0) launch_mask<D, F16, ALIBI, true>(a, grid, block, s);
    else launch_mask<D, F16, ALIBI, false>(a, grid, block, s);
}

template <int D, bool F16>
void launch_alibi(const PrefillArgs &a, dim3 grid, dim3 block, hipStream_t s) {
    if (a.alibi) launch_rope<D, F16, true>(a, grid, block, s);
    else launch_rope<D, F16, false>(a, grid, block, s);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, bool f16, hipStream_t s) {
    const dim3 grid((unsigned)a.num_q_tiles * a.heads_q / a.gqa_pack * a.batch);
    const dim3 block(NTHREADS);
    if (f16) {
        if (head_dim == 128) launch_alibi<128, true>(a, grid, block, s);
        else launch_alibi<64, true>(a, grid, block, s);
    } else {
        if (head_dim == 128) launch_alibi<128, false>(a, grid, block, s);
        else launch_alibi<64, false>(a, grid, block, s);
    }
    return hipGetLastError();
}

}  // namespace fa
