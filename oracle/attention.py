"""fp64 CPU oracle for fused attention -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the benchmark's CPU
baseline may import this module.  The library's product path never routes
through it; the two share no code.

What it computes
----------------
The plain three-step definition of scaled dot-product attention, written out
in float64 with NumPy:

1. scores      S = scale * Q K^T  (+ an ALiBi bias when slopes are given)
   (ops-transformer practice page, jsqmd.com, section 二 "SelfAttention
   baseline and its bottleneck": Attention(Q,K,V) = softmax(QK^T/sqrt(d)) V;
   the naive_attention listing of section 二 "fused computation idea" and the
   BertSelfAttention forward of the agent.csdn.net BERT page, chapter 一,
   take the same three steps: matmul, softmax, matmul.  ALiBi, same page,
   section 三, the part on ALiBi's linear bias: after QK^T/sqrt(d) every pair
   (i, j) gets the bias -m * |i - j|, m a slope that depends on the head.)
2. mask        masked scores are set to -inf, so they vanish after softmax
   (jsqmd.com page, section 二 "causal mask and decode": the upper triangle
   is set to negative infinity; agent.csdn.net BERT page, chapter 四:
   padding positions are masked to negative infinity and so change nothing).
3. softmax     row-wise with the row maximum subtracted before exp
   (hwcomputing.csdn.net page, section 2.2: softmax(x_i) =
   exp(x_i - max x) / sum_j exp(x_j - max x)).
4. output      O = P V and the natural-log log-sum-exp per row,
   LSE_i = m_i + ln(sum_j exp(S_ij - m_i)).

Readings taken where the pages are silent (each also listed in the design
notes):

* scale is one multiplier on QK^T (``softmax_scale``), converted to float64
  from its float32 value;
* valid lengths: query rows ``i >= Lq`` and keys ``j >= Lk`` are not visible
  (the ``actual_seq_q`` / ``actual_seq_kv`` arguments of the BERT page,
  chapter 三 and its closing section);
* causal alignment is bottom-right: query row ``i`` sits at key position
  ``pos_i = i + Lk - Lq`` and sees keys ``j <= pos_i``;
* sliding window ``W >= 1`` keeps keys ``j > pos_i - W`` (W keys including
  the diagonal); ``W = -1`` means no window;
* ALiBi: the page gives no formula for the slopes, so they are an input
  (one per query head); the distance |i - j| is taken between the query's
  key position ``pos_i`` (the causal alignment above) and the key index;
* grouped-query attention maps query head ``h`` to key/value head
  ``h // (Hq // Hkv)`` (contiguous groups); MQA is ``Hkv = 1``;
* a row with no visible key has O = 0 and LSE = -inf (instead of 0/0);
* decode (the BERT page's closing section: the new token attends to all
  cached keys, the cache is not recomputed) is the same computation with a
  single query at position ``L_b - 1`` over cache rows ``0 .. L_b - 1``;
* paged KV cache (GatherPAKVCache, the hwcomputing.csdn.net page, sections
  1.2 and 4.1: the cache rows a query needs are gathered by index rather
  than read as one contiguous block).  The page does not define the index
  structure; the reading here is the paged layout: a pool of pages of
  ``page_size`` consecutive rows each, and per sequence a table whose entry
  ``p`` names the physical page that holds logical rows
  ``p * page_size .. (p + 1) * page_size - 1``.  The attention computed over
  the gathered rows is the decode above, unchanged.  The page's other
  strategies (keeping only "important" rows) change the result and have no
  stated criterion; they are not part of this oracle;
* quantized KV cache (INT8 input with calibration, the jsqmd.com page,
  section 五 on mixed precision; kv_quant_sparse_flash_attention, named in
  the BERT page's preface).  Neither page gives a format or a scale
  convention.  The reading here: each cached K and V element is an 8-bit
  float code in the OCP FP8 E4M3 encoding (E4M3FN: 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN,
  largest finite value 448), with one fp32 scale per KV head for K and one
  for V; the element's value is ``scale * E4M3(code)``.  Attention over the
  dequantized cache is the decode above, unchanged;
* explicit mask (the BERT page: the baseline adds ``mask`` to the scaled
  scores, ``score = score + mask``, chapter 一; its fused replacement passes
  the same tensor as ``attn_mask``, chapter 三; the benchmark builds it as
  [b, 1, 1, n], chapter 五): an additive tensor, broadcast over batch,
  heads and query rows as its shape allows, added to the scaled scores
  before the implicit masks; -inf entries remove a key;
* RoPE (the jsqmd.com page, section 三, rotary position encoding and its
  fusion into attention): the vector at position m is rotated pair by pair,
  each pair of adjacent dimensions (2p, 2p + 1) by its own angle; the page
  gives no angle formula, so the angles enter as tables cos[m, p] and
  sin[m, p] (float32), and only the first ``rotary_dim`` dimensions rotate
  (the page's ``rotary_dim`` argument).  Rotation of (a, b) by an angle with
  cosine c and sine s gives (a c - b s, a s + b c).  Positions follow the
  causal alignment: key j sits at position j and query row i at
  ``i + Lk - Lq``.  Q and K are rotated first and, as the page's separate
  form (apply_rope, then flash_attention) stores them, held in the input
  dtype: each rotated element is rounded to nearest even in bf16 (or fp32).
  Attention over the rotated vectors is unchanged.  When a sequence has
  more query rows than keys (Lq > Lk), the first Lq - Lk query rows sit at
  negative positions, which the tables do not hold; the page defines no
  rotation there.  With RoPE such a row has no visible key: O = 0 and
  LSE = -inf.  (Under the causal mask these rows are empty anyway; the rule
  matters only without it.)

Every function here is pinned in ``tests/test_oracle.py`` against closed
forms, brute force on tiny integer inputs, library routines and invariants.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

NEG_INF = -np.inf


def visible(i: int, j: int, Lq: int, Lk: int, causal: bool, window_left: int) -> bool:
    """Visibility of key ``j`` to query row ``i`` (scalar form of the mask)."""
    if i < 0 or j < 0 or i >= Lq or j >= Lk:
        return False
    pos = i + (Lk - Lq)
    if causal and j > pos:
        return False
    if window_left > 0 and j <= pos - window_left:
        return False
    return True


def visible_matrix(rows: np.ndarray, Nk: int, Lq: int, Lk: int, causal: bool,
                   window_left: int) -> np.ndarray:
    """Boolean mask ``[len(rows), Nk]``: True where key j is visible to row i."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(Nk, dtype=np.int64)[None, :]
    pos = i + (Lk - Lq)
    vis = (i < Lq) & (j < Lk)
    if causal:
        vis &= j <= pos
    if window_left > 0:
        vis &= j > pos - window_left
    return vis


def alibi_bias(rows: np.ndarray, Nk: int, Lq: int, Lk: int, slope: float) -> np.ndarray:
    """ALiBi bias ``[len(rows), Nk]``: -slope * |pos_i - j|, pos_i = i + Lk - Lq."""
    pos = np.asarray(rows, dtype=np.int64)[:, None] + (Lk - Lq)
    j = np.arange(Nk, dtype=np.int64)[None, :]
    return -float(slope) * np.abs(pos - j).astype(np.float64)


def round_to_dtype(x: np.ndarray, dtype: Optional[str]) -> np.ndarray:
    """Round float64 values to the nearest bf16, half ("f16") or fp32 value
    (ties to even), returned as float64; ``dtype=None`` leaves them
    unrounded.  bf16: the significand is scaled to 8 bits and rounded by
    ``rint`` (half to even); half and fp32 by NumPy's casts."""
    x = np.asarray(x, dtype=np.float64)
    if dtype is None:
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def rope_rotate(x: np.ndarray, positions, cos_table, sin_table, rotary_dim: int,
                store: Optional[str] = None) -> np.ndarray:
    """Rotate rows ``x[n, :]`` (float64 copy) at ``positions[n]``: for every
    pair p < rotary_dim / 2, (x[2p], x[2p+1]) -> (x[2p] c - x[2p+1] s,
    x[2p] s + x[2p+1] c) with c = cos_table[pos, p], s = sin_table[pos, p]."""
    x = np.array(x, dtype=np.float64)
    if rotary_dim % 2 or rotary_dim > x.shape[-1]:
        raise ValueError("rotary_dim must be even and at most the row length")
    pos = np.asarray(positions, dtype=np.int64)
    # positions index the tables directly: one outside [0, rows) has no angle
    # (NumPy would wrap a negative index to the end of the table)
    if pos.size and (pos.min() < 0 or pos.max() >= len(cos_table)):
        raise ValueError("RoPE position outside the tables")
    half = rotary_dim // 2
    c = np.asarray(cos_table, dtype=np.float32)[pos][:, :half].astype(np.float64)
    s = np.asarray(sin_table, dtype=np.float32)[pos][:, :half].astype(np.float64)
    a = x[:, 0:rotary_dim:2].copy()
    b = x[:, 1:rotary_dim:2].copy()
    x[:, 0:rotary_dim:2] = round_to_dtype(a * c - b * s, store)
    x[:, 1:rotary_dim:2] = round_to_dtype(a * s + b * c, store)
    return x


def _attend_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 vis: np.ndarray, bias: Optional[np.ndarray] = None):
    """Three-step attention for one (batch, head): q_rows [r, d], k/v [Nk, d]."""
    s = scale * (q_rows @ k.T)                       # step 1
    if bias is not None:
        s = s + bias
    s = np.where(vis, s, NEG_INF)                    # step 2
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    # a row is empty only when no key is visible (m = -inf); NaN inputs on
    # visible keys propagate to the output as the definition implies
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])                  # step 3 (exp(-inf) = 0)
    l = p.sum(axis=1)
    # step 4 sums over visible keys only: keys no row can see are left out of
    # the product, so that their stored values (e.g. NaN padding) never enter
    # it as 0 * NaN.
    cols = vis.any(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (p[:, cols] @ v[cols]) / l[:, None]
        lse = m_safe + np.log(l)
    o[empty] = 0.0
    lse[empty] = NEG_INF
    return o, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: float,
              causal: bool = False, window_left: int = -1,
              seqlens_q: Optional[Sequence[int]] = None,
              seqlens_k: Optional[Sequence[int]] = None,
              rows: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[int]] = None,
              alibi_slopes: Optional[Sequence[float]] = None,
              rope: Optional[tuple] = None,
              attn_mask: Optional[np.ndarray] = None):
    """Reference attention forward.

    q: [B, Nq, Hq, d], k and v: [B, Nk, Hkv, d] (any real dtype; used as
    float64).  Returns ``(O, LSE)`` with O: [B, R, Hq', d] float64 and LSE:
    [B, Hq', R] float64, where R = Nq (or ``len(rows)``) and Hq' = Hq (or
    ``len(heads)``).  ``rows`` / ``heads`` restrict the computation to a
    subset of query rows / heads; each output row depends only on its own
    query and visible keys, so a subset is exact.  ``alibi_slopes`` (one
    float32 value per query head, or None) adds the ALiBi bias to the scores.
    ``rope = (cos_table, sin_table, rotary_dim[, store])`` rotates Q rows
    (at ``i + Lk - Lq``) and K rows (at ``j``) before the scores, rounding
    the rotated elements to ``store`` ("bf16", "f32" or None); only rows
    inside the valid lengths are rotated (the others are never visible).
    A query row at a negative position (``i < Lq - Lk``) has no angle in the
    tables, so under RoPE it sees no key.
    ``attn_mask`` (float array broadcastable to [B, Hq, Nq, Nk]) is added to
    the scaled scores.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    scale = float(np.float32(scale))
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    if alibi_slopes is not None:
        slopes = np.asarray(alibi_slopes, dtype=np.float32).astype(np.float64)
        if slopes.shape != (Hq,):
            raise ValueError("alibi_slopes needs one value per query head")
    if attn_mask is not None:
        attn_mask = np.broadcast_to(np.asarray(attn_mask, dtype=np.float64), (B, Hq, Nq, Nk))
    o = np.zeros((B, len(rows), len(heads), d), dtype=np.float64)
    lse = np.zeros((B, len(heads), len(rows)), dtype=np.float64)
    for b in range(B):
        Lq = Nq if seqlens_q is None else int(seqlens_q[b])
        Lk = Nk if seqlens_k is None else int(seqlens_k[b])
        vis = visible_matrix(rows, Nk, Lq, Lk, causal, window_left)
        if rope is not None:
            cos_t, sin_t, rdim = rope[:3]
            store = rope[3] if len(rope) > 3 else None
            # rows before position 0 have no rotation: they see nothing
            vis[rows + (Lk - Lq) < 0] = False
            # rows inside the valid length, at a position the tables hold
            q_ok = np.flatnonzero((rows < Lq) & (rows + (Lk - Lq) >= 0))
            k_ok = np.arange(min(Lk, Nk))
        for hi, h in enumerate(heads):
            kvh = h // group
            bias = None if alibi_slopes is None else alibi_bias(rows, Nk, Lq, Lk, slopes[h])
            if attn_mask is not None:
                extra = attn_mask[b, h][rows]
                bias = extra if bias is None else bias + extra
            qb, kb = q[b, rows, h, :], k[b, :, kvh, :]
            if rope is not None:
                qb, kb = qb.copy(), kb.copy()
                if len(q_ok):
                    qb[q_ok] = rope_rotate(qb[q_ok], rows[q_ok] + (Lk - Lq), cos_t, sin_t, rdim,
                                           store)
                if len(k_ok):
                    kb[k_ok] = rope_rotate(kb[k_ok], k_ok, cos_t, sin_t, rdim, store)
            ob, lb = _attend_rows(qb, kb, v[b, :, kvh, :], scale, vis, bias)
            o[b, :, hi, :] = ob
            lse[b, hi, :] = lb
    return o, lse


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           seqlens_k: Sequence[int], *, scale: float, window_left: int = -1,
           batches: Optional[Sequence[int]] = None,
           alibi_slopes: Optional[Sequence[float]] = None,
           rope_q: Optional[tuple] = None):
    """Reference single-token decode over a contiguous BSHD cache.

    q: [B, Hq, d]; caches: [B, capacity, Hkv, d]; seqlens_k: [B] (clamped to
    [0, capacity]).  The query of sequence b sits at position L_b - 1 and
    sees cache rows 0 .. L_b - 1 (restricted by the window if W >= 1).
    Returns O: [B', Hq, d] and LSE: [B', Hq] in float64.  Only the valid
    prefix of each cache is read, so poisoned rows beyond it never matter.
    ``rope_q = (cos_table, sin_table, rotary_dim[, store])`` rotates the
    query at its position L_b - 1; cached keys are taken as stored (a decode cache holds
    keys already rotated at their own positions when they were appended).
    """
    B, Hq, d = q.shape
    cap = k_cache.shape[1]
    batches = range(B) if batches is None else batches
    batches = list(batches)
    o = np.zeros((len(batches), Hq, d), dtype=np.float64)
    lse = np.zeros((len(batches), Hq), dtype=np.float64)
    for bi, b in enumerate(batches):
        L = int(min(max(int(seqlens_k[b]), 0), cap))
        qb = q[b]
        if rope_q is not None and L > 0:
            qb = rope_rotate(qb, np.full(qb.shape[0], L - 1), *rope_q)
        ob, lb = attention(qb[None, None], k_cache[b, :L][None], v_cache[b, :L][None],
                           scale=scale, causal=True, window_left=window_left,
                           seqlens_q=[1], seqlens_k=[L], alibi_slopes=alibi_slopes)
        o[bi] = ob[0, 0]
        lse[bi] = lb[0, :, 0]
    return o, lse


def gather_paged(pool: np.ndarray, table_row: Sequence[int], L: int) -> np.ndarray:
    """Logical rows ``0 .. L - 1`` of one sequence from a paged pool.

    pool: [num_pages, page_size, ...]; row j is slot ``j % page_size`` of
    physical page ``table_row[j // page_size]``.
    """
    P = pool.shape[1]
    rows = [pool[int(table_row[j // P]), j % P] for j in range(L)]
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=pool.dtype)
    return np.stack(rows)


def decode_paged(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                 block_table: np.ndarray, seqlens_k: Sequence[int], *, scale: float,
                 window_left: int = -1, batches: Optional[Sequence[int]] = None,
                 alibi_slopes: Optional[Sequence[float]] = None):
    """Reference single-token decode over a paged KV cache.

    q: [B, Hq, d]; pools: [num_pages, page_size, Hkv, d]; block_table:
    [B, pages_per_seq] physical page numbers.  The logical capacity is
    ``pages_per_seq * page_size``; lengths are clamped to [0, capacity].  The
    rows of sequence b are gathered by the table and attended exactly as
    :func:`decode` does for a contiguous cache.  Returns O: [B', Hq, d] and
    LSE: [B', Hq] in float64.
    """
    B, Hq, d = q.shape
    block_table = np.asarray(block_table)
    cap = block_table.shape[1] * k_pool.shape[1]
    batches = list(range(B) if batches is None else batches)
    o = np.zeros((len(batches), Hq, d), dtype=np.float64)
    lse = np.zeros((len(batches), Hq), dtype=np.float64)
    for bi, b in enumerate(batches):
        L = int(min(max(int(seqlens_k[b]), 0), cap))
        kb = gather_paged(k_pool, block_table[b], L)
        vb = gather_paged(v_pool, block_table[b], L)
        ob, lb = attention(q[b][None, None], kb[None], vb[None], scale=scale, causal=True,
                           window_left=window_left, seqlens_q=[1], seqlens_k=[L],
                           alibi_slopes=alibi_slopes)
        o[bi] = ob[0, 0]
        lse[bi] = lb[0, :, 0]
    return o, lse


def fp8_e4m3_value(codes) -> np.ndarray:
    """Exact float64 values of OCP FP8 E4M3 (E4M3FN) codes (uint8).

    Exponent field e (4 bits, bias 7) and mantissa m (3 bits): e = 0 is
    subnormal, m / 8 * 2^-6; otherwise (1 + m / 8) * 2^(e - 7); e = 15 with
    m = 7 is NaN (the format has no infinities).  The sign bit negates.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((c & 0x80) != 0, -mag, mag)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, val)


def dequantize_kv(codes, scales) -> np.ndarray:
    """Values of a quantized K or V cache: codes [..., Hkv, d] (uint8 E4M3),
    scales [Hkv] (float32, one per KV head); value = scale[h] * E4M3(code)."""
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return fp8_e4m3_value(codes) * sc[:, None]
