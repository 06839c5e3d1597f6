// Internal interface between the C-ABI layer (fa_api.cpp) and the kernel
// translation units.  Arguments have already been validated on the host when
// these launchers run.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {

// Kernel arguments for prefill (both dtypes).  Extents are the padded tensor
// extents; per-sequence valid lengths come from the optional device arrays.
struct PrefillArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const int32_t *seqlens_q, *seqlens_k;
    int64_t q_sb, q_ss, q_sh;      // element strides: batch, seq, head
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    int64_t o_sb, o_ss, o_sh;
    int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, group;  // group = heads_q / heads_kv
    int32_t causal, window_left;
    float scale_log2;              // softmax_scale * log2(e)
    float scale;                   // softmax_scale
    int32_t num_q_tiles;           // position blocks per sequence (16-bit path: of 256 / gqa_pack)
    int32_t gqa_pack;              // 16-bit path: query heads of one KV head per workgroup
    int32_t persist_wgs;           // packed 16-bit path: workgroups of the persistent form (0: off)
    const float *alibi;            // ALiBi slopes [heads_q] or null
    const float *rope_cos, *rope_sin;  // RoPE tables [max_pos, rotary_dim / 2], or null
    int32_t rotary_dim;            // 0 = no RoPE
    const void *mask;              // additive mask (dtype of q), or null
    int64_t m_sb, m_sh, m_ss;      // mask element strides: batch, head, query row (key: 1)
};

// K rotation pass (bf16 prefill with RoPE): rows j < Lk of every KV head,
// rotated at position j, into a contiguous [batch, seqlen_k, heads_kv, D] copy.
struct RopeKArgs {
    const void *k;
    void *out;
    const int32_t *seqlens_k;
    int64_t k_sb, k_ss, k_sh;
    int32_t batch, seqlen_k, heads_kv;
    const float *rope_cos, *rope_sin;
    int32_t rotary_dim;
};

struct DecodeArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const int32_t *seqlens_k;
    int64_t q_sb, q_sh;
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    int64_t o_sb, o_sh;
    int32_t batch, heads_q, heads_kv, group, capacity, window_left;
    int32_t chunk;                 // keys per split
    int32_t max_chunks;            // ceil(capacity / chunk)
    int32_t head_groups;           // group / heads_per_wg
    float scale_log2;
    float *ws_o;                   // [batch, heads_q, max_chunks, head_dim] fp32
    float *ws_ml;                  // [batch, heads_q, max_chunks, 2] fp32 (m, l)
    int32_t *ws_items;             // batch > kDecodeRankBatch: item table [1 + batch * max_chunks], else null
    const float *alibi;            // ALiBi slopes [heads_q] or null
    float scale;                   // softmax_scale
    const int32_t *block_table;    // paged cache: [batch, pages_per_seq], or null (contiguous)
    int32_t page_size, pages_per_seq, num_pages;
    int32_t kv_fp8;                // 1: K/V are FP8 E4M3 codes scaled by k_scale / v_scale
    const float *k_scale, *v_scale;  // [heads_kv] (FP8 cache)
    int32_t origin_align;          // chunk grid origin alignment (set by the launcher)
    const float *rope_cos, *rope_sin;  // RoPE tables for the query at L - 1, or null
    int32_t rotary_dim;            // 0 = no RoPE
};

// Each launcher enqueues its kernel(s) and returns the launch status.
// 16-bit prefill (bf16, or IEEE half when f16) and the K rotation pass
hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, bool f16, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, hipStream_t s);
hipError_t launch_rope_k_bf16(const RopeKArgs &a, int head_dim, bool f16, hipStream_t s);
// decode with 16-bit q and o (bf16, or IEEE half when f16)
hipError_t launch_decode_bf16(const DecodeArgs &a, int head_dim, int heads_per_wg, bool f16,
                              hipStream_t s);

// Device address (on `device`) of the file-scope decode scratch array of
// kDecodeScratchBytes, looked up once per device and cached.
hipError_t decode_scratch_address(int device, void **ptr);

// Tile sizes the launchers use (also needed by the host for grid sizing).
constexpr int kPrefillBM = 256;    // query rows per workgroup (bf16 path)
constexpr int kPrefillF32BM = 16;  // query rows per workgroup (fp32 path)
constexpr int kDecodeChunkUnit = 128;  // decode chunks: whole rounds of 4 wavefronts x 16-key tiles
constexpr int kDecodePageUnit = 16;   // paged cache: page sizes are multiples of one tile
constexpr int kDecodeRankBatch = 64;  // decode batches up to this rank their items in the split kernel
// size of the allocation-free decode's scratch array (fa.h: FA_DECODE_NOALLOC_MAX_BYTES)
constexpr size_t kDecodeScratchBytes = 32u << 20;

}  // namespace fa
