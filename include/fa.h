/*
 * fa.h -- C ABI of the fused-attention library for AMD Instinct MI355X
 * (gfx950).  Plain C: callers need neither HIP nor PyTorch headers.
 *
 * The library computes scaled dot-product attention
 *
 *     O = softmax(scale * Q K^T + mask) V,    LSE_i = ln sum_j exp(scale * q_i . k_j)
 *
 * (the attention definition of the ops-transformer practice page on
 * jsqmd.com, section 二 "SelfAttention baseline and its bottleneck") in one
 * fused pass per query tile with a running max / running sum softmax, so the
 * N x N score matrix never reaches device memory (same page, section 二
 * "fused computation idea"; hwcomputing.csdn.net page, sections 2.1-2.2).
 * The sum in LSE runs over visible keys only, in natural log.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; the library
 *   never allocates, frees or keeps device memory between calls.
 * - Strides are in ELEMENTS, not bytes; the innermost (head_dim) stride is 1.
 * - Calls are asynchronous: kernels are enqueued on `hip_stream` (a
 *   hipStream_t passed as void*; NULL = the default stream).  Results are
 *   ready once that stream is synchronised.  Faults inside a kernel surface
 *   at that synchronisation, not as a return code.
 * - Every argument check runs before any HIP call.  A failing check returns
 *   FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED and leaves the outputs
 *   untouched; fa_last_error_message() then describes the problem.
 * - A batch of 0, or a zero query extent, is a valid no-op (FA_OK).
 * - The library has no global state; concurrent calls on different streams
 *   are safe.  The error message buffer is thread-local.
 * - Masking is implicit (no mask tensor is read): the causal mask is applied
 *   by index arithmetic inside the kernel and fully masked tiles are skipped
 *   (jsqmd.com page, section 二 "causal mask and decode"); padding beyond a
 *   valid length is never read (agent.csdn.net BERT page, chapter 四: tiles
 *   whose length is not a multiple of the tile size must not read out of
 *   bounds).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* NULL pointer, bad extent, bad stride, bad scale ... */
    FA_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels implement   */
    FA_ERR_WORKSPACE = 3,     /* decode workspace missing or too small              */
    FA_ERR_HIP = 4            /* the HIP runtime reported an error at launch        */
} fa_status;

typedef enum {
    FA_DTYPE_F32 = 0,         /* fp32 in, fp32 products and accumulation, fp32 out  */
    FA_DTYPE_BF16 = 1,        /* bf16 in, bf16 MFMA with fp32 accumulation, bf16 out */
    FA_DTYPE_F16 = 2          /* IEEE half in, half MFMA / dot products with fp32
                                 accumulation, half out (the FP16 of the pages'
                                 BERT benchmark)                                    */
} fa_dtype;

/* Storage of a decode KV cache (fa_decode_params.kv_format). */
typedef enum {
    FA_KV_PLAIN = 0,          /* K and V in the call's dtype                        */
    FA_KV_FP8_E4M3 = 1        /* K and V as OCP FP8 E4M3 codes, one fp32 scale per
                                 KV head for each (see fa_decode_params)            */
} fa_kv_format;

/*
 * Prefill / encoder attention: fa_prefill_fwd
 * -------------------------------------------
 * Mirrors the fused-operator calls of the pages: flash_attention(query, key,
 * value, causal, softmax_scale) (jsqmd.com page, sections 一 and 二) and
 * flash_attention_score(..., actual_seq_q, actual_seq_kv) with valid lengths
 * instead of a padding mask (agent.csdn.net BERT page, chapter 三 and its
 * closing section on variable-length batches).  Dropout (keep_prob) is not
 * part of the operation.
 *
 * Layout: BSHD by default, [batch, seq, head, dim] (the (N, S, D) input
 * layout of the BERT page, chapter 四), but any layout with a unit dim
 * stride is accepted through the three strides (batch, seq, head); a packed
 * QKV buffer is expressed with three base pointers sharing one seq stride.
 *   q : [batch, seqlen_q, heads_q,  head_dim]
 *   k : [batch, seqlen_k, heads_kv, head_dim]
 *   v : [batch, seqlen_k, heads_kv, head_dim]
 *   o : [batch, seqlen_q, heads_q,  head_dim]   (written; same dtype as q)
 *   lse: contiguous fp32 [batch, heads_q, seqlen_q] (written), or NULL to skip.
 *
 * Visibility of key j to query row i of sequence b, with Lq = seqlens_q[b]
 * (or seqlen_q when NULL) and Lk = seqlens_k[b] (or seqlen_k when NULL),
 * each clamped to [0, extent]:
 *   i < Lq  and  j < Lk
 *   causal:          j <= i + (Lk - Lq)          (bottom-right aligned)
 *   window_left W>0: j >  i + (Lk - Lq) - W      (W keys including the diagonal)
 * A row with no visible key gets O = 0 and LSE = -inf; rows i >= Lq are
 * written as O = 0, LSE = -inf.  Query head h reads key/value head
 * h / (heads_q / heads_kv) (grouped-query attention; MQA when heads_kv = 1).
 *
 * ALiBi (jsqmd.com page, section 三, ALiBi's linear bias): when alibi_slopes
 * is a device fp32 array [heads_q], the score of (i, j) for query head h
 * becomes softmax_scale * q_i . k_j - alibi_slopes[h] * |i + (Lk - Lq) - j|,
 * the bias generated in the kernel (no bias matrix in memory).  The slopes
 * are read on the device, so their values are not validated; NULL = none.
 *
 * RoPE (jsqmd.com page, section 三, rotary position encoding fused into
 * attention): with rotary_dim > 0, every pair of adjacent dims (2p, 2p + 1),
 * p < rotary_dim / 2, of a query or key vector at position m is rotated:
 * (x, y) -> (x c - y s, x s + y c), c = rope_cos[m * rotary_dim / 2 + p],
 * s = rope_sin[...] (device fp32 tables [rope_max_pos, rotary_dim / 2]; the
 * page gives no angle formula, so the caller supplies the tables).  Key j
 * sits at position j, query row i at i + (Lk - Lq).  When a sequence has
 * more query rows than keys (Lq > Lk), its rows i < Lq - Lk sit before
 * position 0, where the tables hold no angle: with RoPE those rows see no
 * key and get O = 0, LSE = -inf (under the causal mask they are empty
 * anyway), and no table entry outside [0, rope_max_pos) is read.  The
 * rotated vectors are rounded to the input dtype before the products, as a
 * separate rotation pass would store them.  Queries are rotated in registers as they are
 * loaded.  Keys: the fp32 path rotates each key tile as it is staged; the
 * bf16 path first rotates K once into `workspace` (a copy of K's valid rows,
 * contiguous [batch, seqlen_k, heads_kv, head_dim]), since its kernel reads
 * every key tile once per 256 query rows and a rotation at each read would
 * cost the matrix wavefronts that many times the vector work.  Requirements:
 * rotary_dim a multiple of 8 and at most head_dim; rope_max_pos >= seqlen_k;
 * tables 16-byte aligned; for bf16, workspace (16-byte aligned, caller-owned,
 * scratch after the call) of at least fa_prefill_workspace_size() bytes.
 * With rotary_dim = 0 the tables and the workspace are ignored.
 *
 * Explicit mask (the BERT page: score = score + mask before softmax in its
 * baseline, chapter 一; passed as attn_mask to the fused operator, chapter
 * 三): attn_mask, when not NULL, is an additive tensor in the call's dtype,
 * read at element b * mask_stride[0] + h * mask_stride[1] + i *
 * mask_stride[2] + j for query head h, row i < seqlen_q and key j <
 * seqlen_k.  A stride of 0 broadcasts that dimension (the page's [b, 1, 1, n]
 * key-padding mask is strides {n, 0, 0, 1}); mask_stride[3] must be 1.  The
 * value is added to softmax_scale * q_i . k_j (after ALiBi, before the
 * implicit masks); -inf removes the key.  Pointer 16-byte aligned;
 * mask_stride[0..2] multiples of 8 elements (bf16, f16) or 4 (fp32).  Values
 * are read on the device and not validated.  The implicit masks stay the
 * cheap way to express causal, window and padding: an explicit mask adds
 * its bytes to every query tile's traffic.  A 16-bit mask with
 * mask_stride[2] == 0 (the same row for every query) is added by the matrix
 * cores and costs less than one whose rows differ.
 *
 * Requirements: head_dim in {64, 128}; heads_q % heads_kv == 0;
 * softmax_scale finite and > 0 (the usual value is 1/sqrt(head_dim));
 * window_left == -1 or >= 1; extents >= 0; seqlens arrays (if given) are
 * device int32 [batch].  Pointers must be 16-byte aligned and strides of
 * batch/seq/head multiples of 8 elements (bf16, f16) or 4 elements (fp32);
 * for bf16 and f16 the seq strides of k and v must be below 2^25 elements.  A request
 * outside these limits returns FA_ERR_UNSUPPORTED or FA_ERR_INVALID_ARG
 * without launching anything.
 */
typedef struct {
    int32_t dtype;                       /* fa_dtype; q, k, v and o share it     */
    int32_t batch;
    int32_t seqlen_q;                    /* padded query extent                  */
    int32_t seqlen_k;                    /* padded key/value extent              */
    int32_t heads_q;
    int32_t heads_kv;
    int32_t head_dim;
    int32_t causal;                      /* 0 or 1                               */
    int32_t window_left;                 /* -1 = none, else W >= 1               */
    float softmax_scale;                 /* multiplier on Q K^T                  */
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;                          /* may be NULL                          */
    const int32_t *seqlens_q;            /* device [batch] or NULL               */
    const int32_t *seqlens_k;            /* device [batch] or NULL               */
    int64_t q_stride[3];                 /* batch, seq, head (elements)          */
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
    const float *alibi_slopes;           /* device fp32 [heads_q] or NULL        */
    const float *rope_cos;               /* device fp32 [rope_max_pos, rotary_dim/2] */
    const float *rope_sin;               /* same shape                           */
    int32_t rotary_dim;                  /* 0 = no RoPE, else k * 8 <= head_dim  */
    int32_t rope_max_pos;                /* rows of the tables (>= seqlen_k)     */
    void *workspace;                     /* bf16 RoPE only: rotated K            */
    int64_t workspace_bytes;
    const void *attn_mask;               /* device additive mask (dtype) or NULL */
    int64_t mask_stride[4];              /* elements: batch, head, row, key (=1) */
} fa_prefill_params;

/*
 * Single-token decode over a KV cache: fa_decode_workspace_size, fa_decode_fwd
 * ---------------------------------------------------------------------------
 * The incremental mode of the BERT page's closing section: the new token's
 * query attends to every cached key/value of its sequence; cached entries
 * are not recomputed.  The caller has already appended the current token's
 * K and V, so sequence b attends to cache rows 0 .. L_b-1 with
 * L_b = seqlens_k[b] clamped to [0, cache_capacity] (device int32 [batch],
 * required).  With window_left = W >= 1 only rows j > L_b - 1 - W are read.
 *   q       : [batch, heads_q, head_dim]          via q_stride (batch, head)
 *   k_cache : [batch, capacity, heads_kv, head_dim] via k_stride (batch, seq, head)
 *   v_cache : same shape, via v_stride
 *   o       : [batch, heads_q, head_dim]          via o_stride (batch, head)
 *   lse     : contiguous fp32 [batch, heads_q], or NULL.
 * Cache rows at or beyond L_b are never read, so they may hold anything.
 * The kernels split each sequence's keys into chunks (split-KV), read every
 * K/V row once for all heads_q / heads_kv query heads of its group, and merge
 * the per-chunk partial results with a log-sum-exp combine pass.
 *
 * chunk_keys: 0 lets the library choose; otherwise a multiple of 128 keys,
 * at most 65536 (other values return FA_ERR_UNSUPPORTED).  Results agree to
 * rounding for every choice.
 *
 * Workspace: fa_decode_workspace_size() reports the bytes fa_decode_fwd needs
 * for this parameter set (it depends on batch, heads, head_dim, capacity and
 * the chunk size only, never on device data).  The caller allocates it
 * (device memory, 16-byte aligned) and passes it in; its contents need no
 * initialisation and are scratch after the call.  Two calls that overlap in
 * time must not share one workspace.
 *
 * ALiBi: as for prefill, with the query at position L_b - 1: the score of
 * cache row j for query head h gets - alibi_slopes[h] * (L_b - 1 - j).
 *
 * Paged KV cache (block_table != NULL): the gather-by-index cache of the
 * hwcomputing.csdn.net page (GatherPAKVCache, sections 1.2 and 4.1), in the
 * paged layout.  k_cache and v_cache are then pools of num_pages pages of
 * page_size rows each, [num_pages, page_size, heads_kv, head_dim] via
 * k_stride / v_stride (page, row, head), and block_table is a device int32
 * array [batch, pages_per_seq]: logical row j of sequence b is row
 * j % page_size of physical page block_table[b * pages_per_seq + j / page_size].
 * The caller owns the pools and the table.  Only the entries of pages that
 * hold rows the query reads are loaded; an entry outside [0, num_pages) is
 * clamped into that range (no read leaves the pools, but that sequence's
 * result is then meaningless).  Requirements: page_size a multiple of 16 in
 * [16, 65536]; pages_per_seq >= 1; num_pages >= 1; cache_capacity <=
 * pages_per_seq * page_size (lengths clamp to cache_capacity); page_size
 * times the row stride of k and v below 2^31 elements.  With block_table
 * NULL, page_size, pages_per_seq and num_pages must be 0.
 *
 * FP8 KV cache (kv_format = FA_KV_FP8_E4M3): the quantized KV cache named on
 * the pages (INT8 input with calibration, jsqmd.com page, section 五;
 * kv_quant_sparse_flash_attention, BERT page preface), which fix no format.
 * Each cached element is one byte, an OCP FP8 E4M3 code (E4M3FN: bias 7, no
 * infinities, S.1111.111 is NaN, largest finite value 448), and its value is
 * k_scale[kvh] * E4M3(code) for K and v_scale[kvh] * E4M3(code) for V, with
 * k_scale and v_scale device fp32 arrays [heads_kv] (read on the device, not
 * validated).  q and o stay bf16.  k/v strides count elements (= bytes) and
 * must be multiples of 16.  Works with the contiguous and the paged layout.
 * With FA_KV_PLAIN, k_scale and v_scale must be NULL.
 *
 * RoPE (as for prefill): with rotary_dim > 0 the query is rotated at its
 * position L_b - 1 as it is loaded.  Cached keys are read as stored: a
 * decode cache holds keys already rotated at their own positions, written
 * when each token was appended.  rope_max_pos >= cache_capacity.
 *
 * Requirements: dtype FA_DTYPE_BF16 or FA_DTYPE_F16 (q, o and a plain
 * cache); head_dim in {64, 128};
 * heads_q % heads_kv == 0; cache_capacity >= 1; softmax_scale finite and > 0.
 */
typedef struct {
    int32_t dtype;                       /* fa_dtype (bf16 or f16)               */
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t head_dim;
    int32_t cache_capacity;              /* rows allocated per sequence          */
    int32_t window_left;                 /* -1 = none, else W >= 1               */
    int32_t chunk_keys;                  /* 0 = library choice, or k * 128       */
    float softmax_scale;
    int32_t reserved0;                   /* must be 0                            */
    const void *q;
    const void *k_cache;
    const void *v_cache;
    void *o;
    float *lse;                          /* may be NULL                          */
    const int32_t *seqlens_k;            /* device [batch], required             */
    int64_t q_stride[2];                 /* batch, head (elements)               */
    int64_t k_stride[3];                 /* batch, seq, head                     */
    int64_t v_stride[3];
    int64_t o_stride[2];                 /* batch, head                          */
    const float *alibi_slopes;           /* device fp32 [heads_q] or NULL        */
    const int32_t *block_table;          /* device [batch, pages_per_seq] or NULL */
    int32_t page_size;                   /* rows per page (paged cache), else 0  */
    int32_t pages_per_seq;               /* block_table row length, else 0       */
    int32_t num_pages;                   /* pages in each pool, else 0           */
    int32_t reserved1;                   /* must be 0                            */
    int32_t kv_format;                   /* fa_kv_format                          */
    int32_t reserved2;                   /* must be 0                            */
    const float *k_scale;                /* device fp32 [heads_kv] (FP8) or NULL */
    const float *v_scale;                /* device fp32 [heads_kv] (FP8) or NULL */
    const float *rope_cos;               /* device fp32 [rope_max_pos, rotary_dim/2] */
    const float *rope_sin;               /* same shape                           */
    int32_t rotary_dim;                  /* 0 = no RoPE, else k * 8 <= head_dim  */
    int32_t rope_max_pos;                /* rows of the tables (>= capacity)     */
} fa_decode_params;

/* Enqueue the prefill forward pass.  Returns FA_OK, FA_ERR_INVALID_ARG,
 * FA_ERR_UNSUPPORTED or FA_ERR_HIP (launch failure). */
fa_status fa_prefill_fwd(const fa_prefill_params *params, void *hip_stream);

/* Bytes of device workspace fa_prefill_fwd needs for `params` (host-only; 0
 * unless bf16 with RoPE, then batch * seqlen_k * heads_kv * head_dim * 2).
 * Writes *bytes and returns FA_OK, or returns an argument error. */
fa_status fa_prefill_workspace_size(const fa_prefill_params *params, size_t *bytes);

/* Bytes of device workspace fa_decode_fwd needs for `params` (host-only
 * computation; no HIP call).  Writes *bytes and returns FA_OK, or returns an
 * argument error without writing. */
fa_status fa_decode_workspace_size(const fa_decode_params *params, size_t *bytes);

/* Enqueue the split-KV decode (two kernels on `hip_stream`).  Returns FA_OK,
 * FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE (NULL workspace or
 * workspace_bytes below fa_decode_workspace_size) or FA_ERR_HIP. */
fa_status fa_decode_fwd(const fa_decode_params *params, void *workspace,
                        size_t workspace_bytes, void *hip_stream);

/*
 * Allocation-free decode: fa_decode_fwd_noalloc
 * ---------------------------------------------
 * For callers that cannot allocate device memory around a decode call:
 * code being captured into a HIP graph, tight serving loops, and harnesses
 * that forbid allocation.  The same operation, parameters and results as
 * fa_decode_fwd (same kernels, bit-identical output), but the partial
 * results live in a device array of the library instead of a caller
 * workspace: FA_DECODE_NOALLOC_MAX_BYTES per GPU, held by each GPU the
 * library runs on from when its code is loaded there until the process
 * ends.  The call allocates and frees nothing.  The first call on a device
 * looks up that device's copy of the array (no allocation; make that first
 * call outside graph capture); later calls only enqueue the two kernels on
 * `hip_stream` (NULL = the default stream of the current device).
 *
 * A parameter set whose fa_decode_workspace_size() exceeds
 * FA_DECODE_NOALLOC_MAX_BYTES returns FA_ERR_WORKSPACE without launching
 * (use fa_decode_fwd with a workspace then).  Nothing in the array needs to
 * start at zero: the combine kernel reads only the partials the split
 * kernel of the same call wrote.  Every call on one GPU shares that GPU's
 * array and overwrites what the previous call left there: calls that
 * overlap in time on one GPU (on different streams, or from host threads
 * without ordering) race and give wrong results; calls ordered on one
 * stream are safe.  Returns what fa_decode_fwd returns, or FA_ERR_HIP when
 * the array's device address cannot be found.
 */
#define FA_DECODE_NOALLOC_MAX_BYTES (32u << 20)
fa_status fa_decode_fwd_noalloc(const fa_decode_params *params, void *hip_stream);

/* Static string naming a status code (never NULL). */
const char *fa_status_str(fa_status status);

/* Thread-local description of the last non-OK return on this thread
 * ("" if none).  Valid until the next library call on the same thread. */
const char *fa_last_error_message(void);

/* ABI version of this header: major * 10000 + minor * 100 + patch. */
int32_t fa_abi_version(void);

#define FA_ABI_VERSION 10700

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
