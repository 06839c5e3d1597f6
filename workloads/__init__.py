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
    """Exact float64 view of stored values (bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
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

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k_cache, self.v_cache, self.seqlens_k):
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


def make_decode(seed: int, B: int, Hq: int, Hkv: int, d: int, capacity: int,
                len_range: tuple, dtype: str = "bf16", *,
                scale: Optional[float] = None, window_left: int = -1,
                lengths: Optional[np.ndarray] = None) -> DecodeProblem:
    """Draw a single-token decode problem over a contiguous BSHD KV cache.

    Lengths are drawn first (uniform in ``len_range``, inclusive) unless given,
    then Q ``[B, Hq, d]``, then per sequence its valid K rows and V rows.
    Cache rows at or beyond the length hold NaN.
    """
    rng = np.random.default_rng(seed)
    if lengths is None:
        lo, hi = len_range
        lengths = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    if dtype == "bf16":
        kc = np.full((B, capacity, Hkv, d), BF16_QNAN, dtype=np.uint16)
        vc = np.full((B, capacity, Hkv, d), BF16_QNAN, dtype=np.uint16)
    else:
        kc = np.full((B, capacity, Hkv, d), np.nan, dtype=np.float32)
        vc = np.full((B, capacity, Hkv, d), np.nan, dtype=np.float32)
    for b in range(B):
        L = int(min(max(lengths[b], 0), capacity))
        kc[b, :L] = _store(rng.standard_normal((L, Hkv, d), dtype=np.float32), dtype)
        vc[b, :L] = _store(rng.standard_normal((L, Hkv, d), dtype=np.float32), dtype)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    return DecodeProblem(dtype, _store(q, dtype), kc, vc, lengths, scale, window_left)


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
