// C-ABI entry points of the fused-attention library (declared in fa.h).
//
// This layer validates every argument on the host before any HIP call,
// converts the public parameter structs into kernel arguments, sizes the
// grids and enqueues the kernels on the caller's stream.  It allocates
// nothing and keeps no state between calls except a thread-local error text.
#include "fa.h"
#include "fa_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

fa_status ok() {
    g_last_error.clear();
    return FA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr float kLog2e = 1.44269504088896340736f;

fa_status check_scale(float scale) {
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(FA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0 (got %g)", (double)scale);
    return FA_OK;
}

fa_status check_strides(const char *name, const int64_t *st, int n, int vec) {
    for (int i = 0; i < n; ++i) {
        if (st[i] < 0) return fail(FA_ERR_INVALID_ARG, "%s_stride[%d] is negative", name, i);
        if (st[i] % vec != 0)
            return fail(FA_ERR_UNSUPPORTED,
                        "%s_stride[%d] = %lld is not a multiple of %d elements (16-byte vector access)",
                        name, i, (long long)st[i], vec);
    }
    return FA_OK;
}

// RoPE tables: rotary_dim a multiple of 8 up to head_dim (whole 16-byte
// pieces of 4 pairs), tables 16-byte aligned and long enough for `positions`.
fa_status check_rope(int rotary_dim, int max_pos, const float *c, const float *sn, int head_dim,
                     int positions, bool need_pointers) {
    if (rotary_dim == 0) return FA_OK;
    if (rotary_dim < 0 || rotary_dim % 8 != 0 || rotary_dim > head_dim)
        return fail(FA_ERR_UNSUPPORTED, "rotary_dim must be 0 or a multiple of 8 up to head_dim (got %d)",
                    rotary_dim);
    if (max_pos < positions)
        return fail(FA_ERR_INVALID_ARG, "rope_max_pos (%d) must cover %d positions", max_pos, positions);
    if (need_pointers) {
        if (!c || !sn) return fail(FA_ERR_INVALID_ARG, "rope_cos and rope_sin must be non-NULL with RoPE");
        if (!aligned16(c) || !aligned16(sn))
            return fail(FA_ERR_UNSUPPORTED, "rope_cos and rope_sin must be 16-byte aligned");
    }
    return FA_OK;
}

#define FA_TRY(expr)                      \
    do {                                  \
        fa_status _s = (expr);            \
        if (_s != FA_OK) return _s;       \
    } while (0)

// Compute units of the device a stream belongs to (cached per device), or -1.
int compute_units(hipStream_t s) {
    static int cached[64];
    int dev = 0;
    if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return -1;
    if (dev < 0 || dev >= 64) return -1;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return -1;
        cached[dev] = n;
    }
    return cached[dev];
}

// Decode: query heads per workgroup (a divisor of the GQA group, at most 4).
int decode_heads_per_wg(int group) {
    if (group % 4 == 0) return 4;
    if (group % 2 == 0) return 2;
    return 1;
}

int decode_chunk(const fa_decode_params *p, int gt) {
    if (p->chunk_keys > 0) return p->chunk_keys;
    // Longest chunk, up to 2048 keys (fewest partials to combine, fewest
    // pipeline fills per key), that still gives about 8 workgroups per CU
    // when every sequence is at capacity; every workgroup streams its chunk
    // with four wavefronts of 16- or 32-key tiles.
    const long long groups = (long long)p->batch * p->heads_kv * (p->heads_q / p->heads_kv / gt);
    int c = 2048;
    while (c > fa::kDecodeChunkUnit && groups * ((p->cache_capacity + c - 1) / c) < 2048) c >>= 1;
    return c;
}

fa_status validate_decode(const fa_decode_params *p) {
    if (!p) return fail(FA_ERR_INVALID_ARG, "params is NULL");
    if (p->dtype != FA_DTYPE_BF16 && p->dtype != FA_DTYPE_F32 && p->dtype != FA_DTYPE_F16)
        return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
    if (p->dtype == FA_DTYPE_F32) return fail(FA_ERR_UNSUPPORTED, "decode supports bf16 and f16 only");
    if (p->batch < 0) return fail(FA_ERR_INVALID_ARG, "batch must be >= 0");
    if (p->heads_q <= 0 || p->heads_kv <= 0)
        return fail(FA_ERR_INVALID_ARG, "heads_q and heads_kv must be >= 1");
    if (p->heads_q % p->heads_kv != 0)
        return fail(FA_ERR_INVALID_ARG, "heads_q (%d) must be a multiple of heads_kv (%d)", p->heads_q,
                    p->heads_kv);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
    if (p->cache_capacity < 1) return fail(FA_ERR_INVALID_ARG, "cache_capacity must be >= 1");
    if (p->window_left == 0 || p->window_left < -1)
        return fail(FA_ERR_INVALID_ARG, "window_left must be -1 or >= 1 (got %d)", p->window_left);
    if (p->chunk_keys != 0 &&
        (p->chunk_keys < 0 || p->chunk_keys % fa::kDecodeChunkUnit != 0 || p->chunk_keys > 65536))
        return fail(FA_ERR_UNSUPPORTED, "chunk_keys must be 0 or a multiple of %d up to 65536 (got %d)",
                    fa::kDecodeChunkUnit, p->chunk_keys);
    if (p->reserved0 != 0 || p->reserved1 != 0 || p->reserved2 != 0)
        return fail(FA_ERR_INVALID_ARG, "reserved0, reserved1 and reserved2 must be 0");
    if (p->kv_format != FA_KV_PLAIN && p->kv_format != FA_KV_FP8_E4M3)
        return fail(FA_ERR_INVALID_ARG, "unknown kv_format %d", p->kv_format);
    if (p->kv_format == FA_KV_PLAIN && (p->k_scale || p->v_scale))
        return fail(FA_ERR_INVALID_ARG, "k_scale and v_scale must be NULL with FA_KV_PLAIN");
    FA_TRY(check_rope(p->rotary_dim, p->rope_max_pos, p->rope_cos, p->rope_sin, p->head_dim,
                      p->cache_capacity, false));
    if (p->block_table) {
        if (p->page_size < fa::kDecodePageUnit || p->page_size > 65536 ||
            p->page_size % fa::kDecodePageUnit != 0)
            return fail(FA_ERR_UNSUPPORTED, "page_size must be a multiple of %d in [%d, 65536] (got %d)",
                        fa::kDecodePageUnit, fa::kDecodePageUnit, p->page_size);
        if (p->pages_per_seq < 1 || p->num_pages < 1)
            return fail(FA_ERR_INVALID_ARG, "pages_per_seq and num_pages must be >= 1 with a block_table");
        if (p->cache_capacity > (int64_t)p->pages_per_seq * p->page_size)
            return fail(FA_ERR_INVALID_ARG, "cache_capacity (%d) exceeds pages_per_seq x page_size (%lld)",
                        p->cache_capacity, (long long)p->pages_per_seq * p->page_size);
        if ((int64_t)p->batch * p->pages_per_seq > 0x7fffffffLL)
            return fail(FA_ERR_UNSUPPORTED, "block_table has more than 2^31 - 1 entries");
    } else if (p->page_size != 0 || p->pages_per_seq != 0 || p->num_pages != 0) {
        return fail(FA_ERR_INVALID_ARG, "page_size, pages_per_seq and num_pages must be 0 without a block_table");
    }
    FA_TRY(check_scale(p->softmax_scale));
    FA_TRY(check_strides("q", p->q_stride, 2, 8));
    // 16-byte vector access: 8 bf16 elements, or 16 FP8 codes
    const int kv_vec = p->kv_format == FA_KV_FP8_E4M3 ? 16 : 8;
    FA_TRY(check_strides("k", p->k_stride, 3, kv_vec));
    FA_TRY(check_strides("v", p->v_stride, 3, kv_vec));
    FA_TRY(check_strides("o", p->o_stride, 2, 1));
    return FA_OK;
}

// Pointer checks, needed to launch but not to size the workspace.
fa_status validate_decode_pointers(const fa_decode_params *p) {
    if (p->batch == 0) return FA_OK;
    if (!p->q || !p->k_cache || !p->v_cache || !p->o || !p->seqlens_k)
        return fail(FA_ERR_INVALID_ARG, "q, k_cache, v_cache, o and seqlens_k must be non-NULL");
    if (!aligned16(p->q) || !aligned16(p->k_cache) || !aligned16(p->v_cache))
        return fail(FA_ERR_UNSUPPORTED, "q, k_cache and v_cache must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(p->o) & 1u) != 0)
        return fail(FA_ERR_INVALID_ARG, "o must be 2-byte aligned");
    if ((reinterpret_cast<uintptr_t>(p->block_table) & 3u) != 0)
        return fail(FA_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
    FA_TRY(check_rope(p->rotary_dim, p->rope_max_pos, p->rope_cos, p->rope_sin, p->head_dim,
                      p->cache_capacity, true));
    if (p->kv_format == FA_KV_FP8_E4M3) {
        if (!p->k_scale || !p->v_scale)
            return fail(FA_ERR_INVALID_ARG, "k_scale and v_scale must be non-NULL with FA_KV_FP8_E4M3");
        if ((reinterpret_cast<uintptr_t>(p->k_scale) & 3u) != 0 ||
            (reinterpret_cast<uintptr_t>(p->v_scale) & 3u) != 0)
            return fail(FA_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
    }
    return FA_OK;
}

// Decode workspace: partial O [batch, heads_q, max_chunks, head_dim] fp32
// (256-byte aligned), then (m, l) pairs [batch, heads_q, max_chunks, 2] fp32,
// then, for batches above kDecodeRankBatch, the item table (int32, count
// first, then up to batch * max_chunks entries).
struct DecodeWsLayout {
    size_t o_bytes, ml_bytes, items_bytes;
    size_t total() const { return o_bytes + ml_bytes + items_bytes; }
};

DecodeWsLayout decode_ws_layout(const fa_decode_params *p, int chunk) {
    const size_t max_chunks = (size_t)(p->cache_capacity + chunk - 1) / chunk;
    const size_t rows = (size_t)p->batch * p->heads_q * max_chunks;
    DecodeWsLayout w;
    w.o_bytes = (rows * p->head_dim * sizeof(float) + 255) & ~(size_t)255;
    w.ml_bytes = (rows * 2 * sizeof(float) + 15) & ~(size_t)15;
    w.items_bytes = p->batch > fa::kDecodeRankBatch ? (1 + (size_t)p->batch * max_chunks) * sizeof(int32_t) : 0;
    return w;
}

size_t decode_ws_bytes(const fa_decode_params *p, int chunk) { return decode_ws_layout(p, chunk).total(); }

// Workspace of a prefill call: the rotated copy of K (bf16 with RoPE only).
size_t prefill_ws_bytes(const fa_prefill_params *p) {
    if (p->rotary_dim == 0 || p->dtype == FA_DTYPE_F32) return 0;
    return (size_t)p->batch * p->seqlen_k * p->heads_kv * p->head_dim * 2;
}

fa_status validate_prefill(const fa_prefill_params *p) {
    if (!p) return fail(FA_ERR_INVALID_ARG, "params is NULL");
    if (p->dtype != FA_DTYPE_BF16 && p->dtype != FA_DTYPE_F32 && p->dtype != FA_DTYPE_F16)
        return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
    if (p->batch < 0 || p->seqlen_q < 0 || p->seqlen_k < 0)
        return fail(FA_ERR_INVALID_ARG, "batch, seqlen_q and seqlen_k must be >= 0");
    if (p->heads_q <= 0 || p->heads_kv <= 0)
        return fail(FA_ERR_INVALID_ARG, "heads_q and heads_kv must be >= 1");
    if (p->heads_q % p->heads_kv != 0)
        return fail(FA_ERR_INVALID_ARG, "heads_q (%d) must be a multiple of heads_kv (%d)", p->heads_q,
                    p->heads_kv);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(FA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
    if (p->causal != 0 && p->causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (p->window_left == 0 || p->window_left < -1)
        return fail(FA_ERR_INVALID_ARG, "window_left must be -1 or >= 1 (got %d)", p->window_left);
    FA_TRY(check_scale(p->softmax_scale));
    const bool half_width = p->dtype != FA_DTYPE_F32;  // bf16 or half
    const int vec = half_width ? 8 : 4;
    FA_TRY(check_strides("q", p->q_stride, 3, vec));
    FA_TRY(check_strides("k", p->k_stride, 3, vec));
    FA_TRY(check_strides("v", p->v_stride, 3, vec));
    FA_TRY(check_strides("o", p->o_stride, 3, vec));
    // the bf16 kernel addresses the rows of one 64-key tile with 32-bit byte offsets
    if (half_width && (p->k_stride[1] >= (1LL << 25) || p->v_stride[1] >= (1LL << 25)))
        return fail(FA_ERR_UNSUPPORTED, "k_stride[1] and v_stride[1] must be below 2^25 elements for bf16 / f16");
    FA_TRY(check_rope(p->rotary_dim, p->rope_max_pos, p->rope_cos, p->rope_sin, p->head_dim,
                      p->seqlen_k, false));
    if (p->attn_mask) {
        if (p->mask_stride[3] != 1) return fail(FA_ERR_UNSUPPORTED, "mask_stride[3] must be 1");
        FA_TRY(check_strides("mask", p->mask_stride, 3, vec));
    }
    // the K rotation pass puts the batch on the second grid axis and a
    // sequence's 16-byte pieces (1024 per workgroup) on the first
    if (p->rotary_dim > 0 && half_width &&
        (p->batch > 65535 || (int64_t)p->seqlen_k * p->heads_kv * (p->head_dim / 8) > (1LL << 34)))
        return fail(FA_ERR_UNSUPPORTED,
                    "RoPE with bf16 / f16 supports a batch up to 65535 and seqlen_k x heads_kv x head_dim up to 2^37");
    return FA_OK;
}

}  // namespace

extern "C" {

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

const char *fa_status_str(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_HIP: return "FA_ERR_HIP";
    }
    return "FA_ERR_UNKNOWN";
}

const char *fa_last_error_message(void) { return g_last_error.c_str(); }

fa_status fa_prefill_workspace_size(const fa_prefill_params *p, size_t *bytes) {
    if (!bytes) return fail(FA_ERR_INVALID_ARG, "bytes is NULL");
    FA_TRY(validate_prefill(p));
    *bytes = prefill_ws_bytes(p);
    return ok();
}

fa_status fa_prefill_fwd(const fa_prefill_params *p, void *hip_stream) {
    FA_TRY(validate_prefill(p));
    if (p->batch == 0 || p->seqlen_q == 0) return ok();
    if (!p->q || !p->o) return fail(FA_ERR_INVALID_ARG, "q and o must be non-NULL");
    if (p->seqlen_k > 0 && (!p->k || !p->v))
        return fail(FA_ERR_INVALID_ARG, "k and v must be non-NULL when seqlen_k > 0");
    if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->o))
        return fail(FA_ERR_UNSUPPORTED, "q, k, v and o must be 16-byte aligned");
    FA_TRY(check_rope(p->rotary_dim, p->rope_max_pos, p->rope_cos, p->rope_sin, p->head_dim,
                      p->seqlen_k, true));
    if (p->attn_mask && !aligned16(p->attn_mask))
        return fail(FA_ERR_UNSUPPORTED, "attn_mask must be 16-byte aligned");
    const size_t ws_need = prefill_ws_bytes(p);
    if (ws_need > 0 && p->seqlen_k > 0) {
        if (!p->workspace) return fail(FA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", ws_need);
        if (!aligned16(p->workspace)) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        if (p->workspace_bytes < 0 || (size_t)p->workspace_bytes < ws_need)
            return fail(FA_ERR_WORKSPACE, "workspace too small: %lld < %zu bytes",
                        (long long)p->workspace_bytes, ws_need);
    }

    fa::PrefillArgs a{};
    a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.lse = p->lse;
    a.seqlens_q = p->seqlens_q; a.seqlens_k = p->seqlens_k;
    a.q_sb = p->q_stride[0]; a.q_ss = p->q_stride[1]; a.q_sh = p->q_stride[2];
    a.k_sb = p->k_stride[0]; a.k_ss = p->k_stride[1]; a.k_sh = p->k_stride[2];
    a.v_sb = p->v_stride[0]; a.v_ss = p->v_stride[1]; a.v_sh = p->v_stride[2];
    a.o_sb = p->o_stride[0]; a.o_ss = p->o_stride[1]; a.o_sh = p->o_stride[2];
    a.batch = p->batch; a.seqlen_q = p->seqlen_q; a.seqlen_k = p->seqlen_k;
    a.heads_q = p->heads_q; a.heads_kv = p->heads_kv; a.group = p->heads_q / p->heads_kv;
    a.causal = p->causal; a.window_left = p->window_left;
    a.scale = p->softmax_scale;
    a.scale_log2 = p->softmax_scale * kLog2e;
    a.alibi = p->alibi_slopes;
    if (p->rotary_dim > 0) {
        a.rope_cos = p->rope_cos; a.rope_sin = p->rope_sin; a.rotary_dim = p->rotary_dim;
    }
    a.mask = p->attn_mask;
    a.m_sb = p->mask_stride[0]; a.m_sh = p->mask_stride[1]; a.m_ss = p->mask_stride[2];
    const bool f16 = p->dtype == FA_DTYPE_F16;
    // bf16 at d = 128: the query heads of a GQA group share a workgroup, up to
    // the 8 wavefronts of 32 rows (gcd(group, 8) heads of 256 / gcd positions)
    a.gqa_pack = 1;
    if (p->dtype == FA_DTYPE_BF16 && p->head_dim == 128)
        while (a.gqa_pack < 8 && a.group % (2 * a.gqa_pack) == 0) a.gqa_pack *= 2;
    const int bm = p->dtype != FA_DTYPE_F32 ? fa::kPrefillBM / a.gqa_pack : fa::kPrefillF32BM;
    a.num_q_tiles = (p->seqlen_q + bm - 1) / bm;
    if ((int64_t)a.num_q_tiles * a.heads_q * a.batch > 0x7fffffffLL)
        return fail(FA_ERR_UNSUPPORTED, "grid too large");

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    // packed GQA without biases: one workgroup per CU walks the work items
    // (the kernel holds one workgroup per CU)
    if (a.gqa_pack > 1 && !p->alibi_slopes && p->rotary_dim == 0 && !p->attn_mask) {
        const int cus = compute_units(s);
        if (cus < 0) return fail(FA_ERR_HIP, "cannot query the device of the stream");
        a.persist_wgs = cus;
    }
    if (ws_need > 0 && p->seqlen_k > 0) {
        // bf16 with RoPE: rotate K once into the workspace, then attend to it
        fa::RopeKArgs r{};
        r.k = p->k; r.out = p->workspace; r.seqlens_k = p->seqlens_k;
        r.k_sb = p->k_stride[0]; r.k_ss = p->k_stride[1]; r.k_sh = p->k_stride[2];
        r.batch = p->batch; r.seqlen_k = p->seqlen_k; r.heads_kv = p->heads_kv;
        r.rope_cos = p->rope_cos; r.rope_sin = p->rope_sin; r.rotary_dim = p->rotary_dim;
        const hipError_t er = fa::launch_rope_k_bf16(r, p->head_dim, f16, s);
        if (er != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(er));
        a.k = p->workspace;
        a.k_sb = (int64_t)p->seqlen_k * p->heads_kv * p->head_dim;
        a.k_ss = (int64_t)p->heads_kv * p->head_dim;
        a.k_sh = p->head_dim;
    }
    const hipError_t e = p->dtype != FA_DTYPE_F32 ? fa::launch_prefill_bf16(a, p->head_dim, f16, s)
                                                  : fa::launch_prefill_f32(a, p->head_dim, s);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

fa_status fa_decode_workspace_size(const fa_decode_params *p, size_t *bytes) {
    if (!bytes) return fail(FA_ERR_INVALID_ARG, "bytes is NULL");
    FA_TRY(validate_decode(p));
    const int gt = decode_heads_per_wg(p->heads_q / p->heads_kv);
    *bytes = p->batch == 0 ? 0 : decode_ws_bytes(p, decode_chunk(p, gt));
    return ok();
}

}  // extern "C"

namespace {

// Limits of the launch itself (after validate_decode and
// validate_decode_pointers, before any HIP call).
fa_status validate_decode_launch(const fa_decode_params *p) {
    const int group = p->heads_q / p->heads_kv;
    const int gt = decode_heads_per_wg(group);
    const int chunk = decode_chunk(p, gt);
    const int max_chunks = (p->cache_capacity + chunk - 1) / chunk;
    // the split kernel addresses the rows of one sequence (one page when
    // paged) with 32-bit byte offsets
    const int64_t rows_addressed = p->block_table ? p->page_size : p->cache_capacity;
    const int64_t elem_bytes = p->kv_format == FA_KV_FP8_E4M3 ? 1 : 2;
    if (rows_addressed * std::max(p->k_stride[1], p->v_stride[1]) * elem_bytes > 0xffffffffLL)
        return fail(FA_ERR_UNSUPPORTED, p->block_table ? "page_size x seq stride exceeds 4 GiB per page"
                                                       : "cache_capacity x seq stride exceeds 4 GiB per sequence");
    if ((int64_t)p->batch * p->heads_q > 0x7fffffffLL ||
        (int64_t)p->heads_kv * (group / gt) * p->batch * max_chunks > 0x7fffffffLL)
        return fail(FA_ERR_UNSUPPORTED, "grid too large");
    return FA_OK;
}

// Enqueue the decode of validated parameters (batch > 0) with `workspace`
// (device memory of at least decode_ws_bytes bytes, 16-byte aligned).
fa_status decode_enqueue(const fa_decode_params *p, void *workspace, void *hip_stream) {
    const int group = p->heads_q / p->heads_kv;
    const int gt = decode_heads_per_wg(group);
    const int chunk = decode_chunk(p, gt);
    const int max_chunks = (p->cache_capacity + chunk - 1) / chunk;

    fa::DecodeArgs a{};
    a.q = p->q; a.k = p->k_cache; a.v = p->v_cache; a.o = p->o; a.lse = p->lse;
    a.seqlens_k = p->seqlens_k;
    a.q_sb = p->q_stride[0]; a.q_sh = p->q_stride[1];
    a.k_sb = p->k_stride[0]; a.k_ss = p->k_stride[1]; a.k_sh = p->k_stride[2];
    a.v_sb = p->v_stride[0]; a.v_ss = p->v_stride[1]; a.v_sh = p->v_stride[2];
    a.o_sb = p->o_stride[0]; a.o_sh = p->o_stride[1];
    a.batch = p->batch; a.heads_q = p->heads_q; a.heads_kv = p->heads_kv; a.group = group;
    a.capacity = p->cache_capacity; a.window_left = p->window_left;
    a.chunk = chunk; a.max_chunks = max_chunks; a.head_groups = group / gt;
    a.scale_log2 = p->softmax_scale * kLog2e;
    a.scale = p->softmax_scale;
    a.alibi = p->alibi_slopes;
    a.block_table = p->block_table;
    a.page_size = p->page_size; a.pages_per_seq = p->pages_per_seq; a.num_pages = p->num_pages;
    a.kv_fp8 = p->kv_format == FA_KV_FP8_E4M3;
    a.k_scale = p->k_scale; a.v_scale = p->v_scale;
    if (p->rotary_dim > 0) {
        a.rope_cos = p->rope_cos; a.rope_sin = p->rope_sin; a.rotary_dim = p->rotary_dim;
    }
    const DecodeWsLayout w = decode_ws_layout(p, chunk);
    a.ws_o = static_cast<float *>(workspace);
    a.ws_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + w.o_bytes);
    a.ws_items = w.items_bytes ? reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + w.o_bytes +
                                                             w.ml_bytes)
                               : nullptr;

    const hipError_t e = fa::launch_decode_bf16(a, p->head_dim, gt, p->dtype == FA_DTYPE_F16,
                                                static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

fa_status fa_decode_fwd(const fa_decode_params *p, void *workspace, size_t workspace_bytes,
                        void *hip_stream) {
    FA_TRY(validate_decode(p));
    FA_TRY(validate_decode_pointers(p));
    if (p->batch == 0) return ok();
    const size_t need = decode_ws_bytes(p, decode_chunk(p, decode_heads_per_wg(p->heads_q / p->heads_kv)));
    if (!workspace) return fail(FA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (!aligned16(workspace)) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    FA_TRY(validate_decode_launch(p));
    return decode_enqueue(p, workspace, hip_stream);
}

fa_status fa_decode_fwd_noalloc(const fa_decode_params *p, void *hip_stream) {
    static_assert(FA_DECODE_NOALLOC_MAX_BYTES == fa::kDecodeScratchBytes, "scratch size");
    FA_TRY(validate_decode(p));
    FA_TRY(validate_decode_pointers(p));
    if (p->batch == 0) return ok();
    const size_t need = decode_ws_bytes(p, decode_chunk(p, decode_heads_per_wg(p->heads_q / p->heads_kv)));
    if (need > fa::kDecodeScratchBytes)
        return fail(FA_ERR_WORKSPACE,
                    "this decode needs %zu bytes of scratch, more than the %zu-byte device array of "
                    "fa_decode_fwd_noalloc; call fa_decode_fwd with a workspace instead",
                    need, (size_t)fa::kDecodeScratchBytes);
    FA_TRY(validate_decode_launch(p));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "cannot find the stream's device: %s", hipGetErrorString(e));
    void *scratch = nullptr;
    e = fa::decode_scratch_address(dev, &scratch);
    if (e != hipSuccess)
        return fail(FA_ERR_HIP, "device %d: no address for the decode scratch array: %s", dev,
                    hipGetErrorString(e));
    return decode_enqueue(p, scratch, hip_stream);
}

}  // extern "C"
