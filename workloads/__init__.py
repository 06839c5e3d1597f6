"""Seeded synthetic inputs for the attention path.

This module only draws numbers and stores them: it holds none of the
attention arithmetic.  Both the fp64 oracle (through the tests) and the
HIP path (through the tests and the benchmark) are fed from here, so the
two sides see exactly the same bits.

Conventions
-----------
* Generator: ``numpy.random.default_rng(seed)`` (PCG64).
* Draw order: valid lengths first, then Q, K, V, each as
  ``standard_normal(..., float32)`` in BSHD order ``[batch, seq, head, dim]``.
* bf16 tensors are produced by round-to-nearest-even of the fp32 draws and
  kept as raw ``uint16`` bit patterns; :func:`bf16_bits_to_f32` decodes them
  exactly.
* Decode caches: rows at or beyond a sequence's length are filled with a
  quiet NaN so that any read past the valid prefix poisons the output.

The shapes of the five named workloads follow the attention problem
statement of the pages: a tiny fp32 single-head case, a BERT-base encoder
(12 heads, d=64, seq 512, per-sequence valid lengths), a 7B-decoder-shaped
causal prefill (32 heads, d=128, N=8192), a GQA causal prefill with a
1024-key sliding window, and a single-token decode over a KV cache.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)
F16_QNAN = np.uint16(0x7E00)


# --------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as ``uint16``.  NaN stays a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding_bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding_bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (bf16 bits, half bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        # IEEE half by NumPy's round-to-nearest-even cast, kept as bit patterns
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# Generated problems
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillProblem:
    dtype: str                       # "bf16" or "f32"
    q: np.ndarray                    # [B, Nq, Hq, d]  (uint16 bits or float32)
    k: np.ndarray                    # [B, Nk, Hkv, d]
    v: np.ndarray                    # [B, Nk, Hkv, d]
    scale: float
    causal: bool = False
    window_left: int = -1
    seqlens_q: Optional[np.ndarray] = None   # int32 [B] or None
    seqlens_k: Optional[np.ndarray] = None   # int32 [B] or None

    @property
    def shape(self):
        B, Nq, Hq, d = self.q.shape
        return B, Nq, self.k.shape[1], Hq, self.k.shape[2], d

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k, self.v, self.seqlens_q, self.seqlens_k):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


@dataclasses.dataclass
class DecodeProblem:
    dtype: str
    q: np.ndarray                    # [B, Hq, d]
    k_cache: np.ndarray              # [B, capacity, Hkv, d]
    v_cache: np.ndarray              # [B, capacity, Hkv, d]
    seqlens_k: np.ndarray            # int32 [B]
    scale: float
    window_left: int = -1
    kv_dtype: Optional[str] = None   # None: caches in dtype; "fp8_e4m3": uint8 codes
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (fp8 caches)
    v_scale: Optional[np.ndarray] = None

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k_cache, self.v_cache, self.seqlens_k, self.k_scale, self.v_scale):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def make_prefill(seed: int, B: int, Nq: int, Nk: int, Hq: int, Hkv: int,
                 d: int, dtype: str = "bf16", *, causal: bool = False,
                 window_left: int = -1, scale: Optional[float] = None,
                 seqlens_k_range: Optional[tuple] = None,
                 seqlens_q_equal_k: bool = False,
                 poison_padding: bool = False) -> PrefillProblem:
    """Draw a prefill problem.

    ``seqlens_k_range=(lo, hi)`` draws per-sequence key lengths uniformly in
    ``[lo, hi]`` (inclusive) before Q, K, V.  With ``seqlens_q_equal_k`` the
    same lengths are also used for the queries.  ``poison_padding`` fills
    key/value rows at or beyond the key length (and query rows at or beyond
    the query length) with NaN after drawing.
    """
    rng = np.random.default_rng(seed)
    seqlens_k = None
    if seqlens_k_range is not None:
        lo, hi = seqlens_k_range
        seqlens_k = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    q = rng.standard_normal((B, Nq, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, Nk, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, Nk, Hkv, d), dtype=np.float32)
    seqlens_q = seqlens_k.copy() if (seqlens_q_equal_k and seqlens_k is not None) else None
    if poison_padding:
        if seqlens_k is not None:
            for b in range(B):
                k[b, seqlens_k[b]:] = np.nan
                v[b, seqlens_k[b]:] = np.nan
        if seqlens_q is not None:
            for b in range(B):
                q[b, seqlens_q[b]:] = np.nan
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    return PrefillProblem(dtype, _store(q, dtype), _store(k, dtype), _store(v, dtype),
                          scale, causal, window_left, seqlens_q, seqlens_k)


FP8_E4M3_QNAN = np.uint8(0x7F)
FP8_E4M3_MAX = 448.0


def f32_to_fp8_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to OCP FP8 E4M3 codes (nearest, ties to even), by
    torch's float8_e4m3fn cast.  Inputs must lie within +-448."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _draw_decode(rng, B, Hq, Hkv, d, capacity, len_range, lengths):
    """Lengths (unless given), then Q, then per sequence its K rows and V rows."""
    if lengths is None:
        lo, hi = len_range
        lengths = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    rows_k, rows_v = [], []
    for b in range(B):
        L = int(min(max(lengths[b], 0), capacity))
        rows_k.append(rng.standard_normal((L, Hkv, d), dtype=np.float32))
        rows_v.append(rng.standard_normal((L, Hkv, d), dtype=np.float32))
    return lengths, q, rows_k, rows_v


def _store_rows(rows, dtype, kv_dtype, Hkv):
    """Stored form of every sequence's rows, the NaN fill value and the
    per-KV-head scales (fp8: scale = max |x| over the head's rows / 448, in
    fp32, and codes = E4M3(x / scale))."""
    if kv_dtype is None:
        fill = {"bf16": BF16_QNAN, "f16": F16_QNAN}.get(dtype, np.float32(np.nan))
        return [_store(r, dtype) for r in rows], fill, None
    if kv_dtype != "fp8_e4m3":
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    amax = np.zeros(Hkv, dtype=np.float32)
    for r in rows:
        if r.shape[0]:
            amax = np.maximum(amax, np.abs(r).max(axis=(0, 2)))
    scales = np.where(amax > 0, amax / np.float32(FP8_E4M3_MAX), np.float32(1.0)).astype(np.float32)
    codes = [f32_to_fp8_e4m3_codes(np.clip(r / scales[None, :, None], -FP8_E4M3_MAX, FP8_E4M3_MAX))
             for r in rows]
    return codes, FP8_E4M3_QNAN, scales


def make_decode(seed: int, B: int, Hq: int, Hkv: int, d: int, capacity: int,
                len_range: tuple, dtype: str = "bf16", *,
                scale: Optional[float] = None, window_left: int = -1,
                lengths: Optional[np.ndarray] = None,
                kv_dtype: Optional[str] = None) -> DecodeProblem:
    """Draw a single-token decode problem over a contiguous BSHD KV cache.

    Lengths are drawn first (uniform in ``len_range``, inclusive) unless given,
    then Q ``[B, Hq, d]``, then per sequence its valid K rows and V rows.
    Cache rows at or beyond the length hold NaN.  ``kv_dtype="fp8_e4m3"``
    stores K and V as E4M3 codes with one fp32 scale per KV head each (the
    same draws, so the same logical cache up to quantization); Q stays in
    ``dtype``.
    """
    rng = np.random.default_rng(seed)
    lengths, q, rows_k, rows_v = _draw_decode(rng, B, Hq, Hkv, d, capacity, len_range, lengths)
    sk, fill, k_scale = _store_rows(rows_k, dtype, kv_dtype, Hkv)
    sv, _, v_scale = _store_rows(rows_v, dtype, kv_dtype, Hkv)
    kc = np.full((B, capacity, Hkv, d), fill, dtype=np.asarray(fill).dtype)
    vc = np.full((B, capacity, Hkv, d), fill, dtype=np.asarray(fill).dtype)
    for b in range(B):
        kc[b, :sk[b].shape[0]] = sk[b]
        vc[b, :sv[b].shape[0]] = sv[b]
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    return DecodeProblem(dtype, _store(q, dtype), kc, vc, lengths, scale, window_left,
                         kv_dtype, k_scale, v_scale)


@dataclasses.dataclass
class PagedDecodeProblem:
    dtype: str
    q: np.ndarray                    # [B, Hq, d]
    k_pool: np.ndarray               # [num_pages, page_size, Hkv, d]
    v_pool: np.ndarray               # [num_pages, page_size, Hkv, d]
    block_table: np.ndarray          # int32 [B, pages_per_seq]
    seqlens_k: np.ndarray            # int32 [B]
    scale: float
    window_left: int = -1
    kv_dtype: Optional[str] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None

    @property
    def page_size(self) -> int:
        return self.k_pool.shape[1]

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k_pool, self.v_pool, self.block_table, self.seqlens_k,
                  self.k_scale, self.v_scale):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()

    @property
    def capacity(self) -> int:
        return self.block_table.shape[1] * self.page_size


def make_decode_paged(seed: int, B: int, Hq: int, Hkv: int, d: int, capacity: int,
                      len_range: tuple, page_size: int, dtype: str = "bf16", *,
                      scale: Optional[float] = None, window_left: int = -1,
                      lengths: Optional[np.ndarray] = None,
                      spare_pages: int = 1, kv_dtype: Optional[str] = None) -> PagedDecodeProblem:
    """Draw a single-token decode problem over a paged KV cache.

    The draws are those of :func:`make_decode` with the same arguments
    (lengths, Q, then per sequence its K rows and V rows), so both layouts hold
    the same logical cache for one seed.  Each sequence's rows then go, page by
    page in logical order, into physical pages taken from a seeded random
    permutation of the pool (a fragmented pool).  ``pages_per_seq`` is
    ``ceil(capacity / page_size)``.  The pool holds the pages in use plus
    ``spare_pages`` (>= 1) pages of NaN; slots past a sequence's length in its
    last page hold NaN, and every table entry past the pages in use names the
    first spare page, so any read the lengths do not allow poisons the output.
    """
    if spare_pages < 1:
        raise ValueError("spare_pages must be >= 1")
    rng = np.random.default_rng(seed)
    lengths, q, rows_k, rows_v = _draw_decode(rng, B, Hq, Hkv, d, capacity, len_range, lengths)
    sk, fill, k_scale = _store_rows(rows_k, dtype, kv_dtype, Hkv)
    sv, _, v_scale = _store_rows(rows_v, dtype, kv_dtype, Hkv)
    P = int(page_size)
    per_seq = -(-capacity // P)
    used = [-(-r.shape[0] // P) for r in sk]
    n_pages = sum(used) + spare_pages
    kp = np.full((n_pages, P, Hkv, d), fill, dtype=np.asarray(fill).dtype)
    vp = np.full((n_pages, P, Hkv, d), fill, dtype=np.asarray(fill).dtype)
    order = rng.permutation(n_pages).astype(np.int32)
    spare = order[sum(used)]
    table = np.full((B, per_seq), spare, dtype=np.int32)
    nxt = 0
    for b in range(B):
        L = sk[b].shape[0]
        for pg in range(used[b]):
            phys = order[nxt]
            nxt += 1
            table[b, pg] = phys
            n = min(P, L - pg * P)
            kp[phys, :n] = sk[b][pg * P:pg * P + n]
            vp[phys, :n] = sv[b][pg * P:pg * P + n]
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    return PagedDecodeProblem(dtype, _store(q, dtype), kp, vp, table, lengths, scale, window_left,
                              kv_dtype, k_scale, v_scale)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
WORKLOADS = {
    1: dict(name="tiny_fp32", kind="prefill", seed=1, B=1, Nq=128, Nk=128, Hq=1, Hkv=1,
            d=64, dtype="f32"),
    2: dict(name="bert_base_varlen", kind="prefill", seed=2, B=8, Nq=512, Nk=512, Hq=12,
            Hkv=12, d=64, dtype="bf16", seqlens_k_range=(128, 512)),
    3: dict(name="decoder7b_causal_8k", kind="prefill", seed=3, B=1, Nq=8192, Nk=8192,
            Hq=32, Hkv=32, d=128, dtype="bf16", causal=True),
    4: dict(name="gqa_causal_window1024", kind="prefill", seed=4, B=2, Nq=4096, Nk=4096,
            Hq=32, Hkv=8, d=128, dtype="bf16", causal=True, window_left=1024),
    5: dict(name="decode_gqa_kvcache", kind="decode", seed=5, B=64, Hq=32, Hkv=8, d=128,
            capacity=8192, len_range=(512, 8192), dtype="bf16"),
}


def make_workload(idx: int):
    """Generate one of the five named workloads at its full size."""
    w = dict(WORKLOADS[idx])
    kind = w.pop("kind")
    w.pop("name")
    seed = w.pop("seed")
    if kind == "prefill":
        return make_prefill(seed, w.pop("B"), w.pop("Nq"), w.pop("Nk"), w.pop("Hq"),
                            w.pop("Hkv"), w.pop("d"), w.pop("dtype"), **w)
    return make_decode(seed, w.pop("B"), w.pop("Hq"), w.pop("Hkv"), w.pop("d"),
                       w.pop("capacity"), w.pop("len_range"), w.pop("dtype"), **w)


def make_workload_paged(idx: int, page_size: int,
                        kv_dtype: Optional[str] = None) -> PagedDecodeProblem:
    """A named decode workload with its cache in a paged pool (same logical
    rows as :func:`make_workload` for that index)."""
    w = dict(WORKLOADS[idx])
    if w.pop("kind") != "decode":
        raise ValueError("only decode workloads have a paged form")
    w.pop("name")
    return make_decode_paged(w.pop("seed"), w.pop("B"), w.pop("Hq"), w.pop("Hkv"), w.pop("d"),
                             w.pop("capacity"), w.pop("len_range"), page_size, w.pop("dtype"),
                             kv_dtype=kv_dtype, **w)


def make_workload_fp8(idx: int) -> DecodeProblem:
    """A named decode workload with an FP8 E4M3 cache (same draws)."""
    w = dict(WORKLOADS[idx])
    if w.pop("kind") != "decode":
        raise ValueError("only decode workloads have an FP8 cache")
    w.pop("name")
    return make_decode(w.pop("seed"), w.pop("B"), w.pop("Hq"), w.pop("Hkv"), w.pop("d"),
                       w.pop("capacity"), w.pop("len_range"), w.pop("dtype"),
                       kv_dtype="fp8_e4m3", **w)
