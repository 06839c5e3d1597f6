"""Fused attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``include/fa.h`` (``libfa.so``).
PyTorch only supplies device memory and the current HIP stream; every step
of the computation runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: without the built library, or with tensors that are not
on a GPU, the calls raise.

    o, lse = prefill(q, k, v, causal=True)            # q: [B, Nq, Hq, d]
    o, lse = decode(q, k_cache, v_cache, seqlens_k)   # q: [B, Hq, d]

Both mirror the pages' fused operators: ``flash_attention(query, key, value,
causal, softmax_scale)`` (jsqmd.com ops-transformer practice page, sections
一 and 二) with valid lengths in place of a padding mask (``actual_seq_q`` /
``actual_seq_kv`` of the agent.csdn.net BERT page, chapter 三), and the
incremental decode of the BERT page's closing section.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

from . import _lib
from ._lib import FAError  # noqa: F401

__all__ = ["prefill", "prefill_workspace_size", "decode", "decode_noalloc",
           "decode_workspace_size", "FAError", "load_library"]


def load_library():
    """Load ``libfa.so`` (raises ImportError if it has not been built)."""
    return _lib.load()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.FA_DTYPE_BF16
    if t.dtype == torch.float16:
        return _lib.FA_DTYPE_F16
    if t.dtype == torch.float32:
        return _lib.FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")


def _require_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on a GPU device (no CPU fallback exists)")


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _seqlens(x, B, device):
    torch = _torch()
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        x = torch.tensor(list(x), dtype=torch.int32)
    x = x.to(device=device, dtype=torch.int32).contiguous()
    if x.numel() != B:
        raise ValueError(f"seqlens must have {B} entries")
    return x


def _slopes(x, H, device):
    torch = _torch()
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        x = torch.tensor(list(x), dtype=torch.float32)
    x = x.to(device=device, dtype=torch.float32).contiguous()
    if x.numel() != H:
        raise ValueError(f"alibi_slopes must have {H} entries (one per query head)")
    return x


def _rope(rope_cos, rope_sin, rotary_dim, device):
    """(cos, sin, rotary_dim, max_pos) device tables, or None without RoPE."""
    torch = _torch()
    if rope_cos is None and rope_sin is None:
        return None
    if rope_cos is None or rope_sin is None:
        raise ValueError("RoPE needs both rope_cos and rope_sin")
    c = rope_cos.to(device=device, dtype=torch.float32).contiguous()
    s = rope_sin.to(device=device, dtype=torch.float32).contiguous()
    if c.dim() != 2 or c.shape != s.shape:
        raise ValueError("rope_cos and rope_sin must both be [max_pos, rotary_dim / 2]")
    rdim = 2 * c.shape[1] if rotary_dim is None else int(rotary_dim)
    if rdim > 2 * c.shape[1]:
        raise ValueError("rotary_dim exceeds the tables' width")
    # the kernels index the tables with a row stride of rotary_dim / 2
    if 2 * c.shape[1] != rdim:
        c, s = c[:, :rdim // 2].contiguous(), s[:, :rdim // 2].contiguous()
    return c, s, rdim, c.shape[0]


def _mask(m, dtype, shape, device):
    """The mask as a [B, Hq, Nq, Nk] view in q's dtype: broadcast dims keep
    stride 0, keys are contiguous, and the other strides are whole 16-byte
    vectors (rows are padded in a copy when they are not)."""
    torch = _torch()
    if m is None:
        return None
    m = m.to(device=device, dtype=dtype)
    while m.dim() < 4:
        m = m.unsqueeze(0)
    m = m.expand(*shape)
    vec = 16 // m.element_size()
    if m.stride(3) != 1 or any(st % vec for st in m.stride()[:3]) or m.data_ptr() % 16:
        Nk = shape[3]
        pad = (Nk + vec - 1) // vec * vec
        keep = [sz if st != 0 else 1 for sz, st in zip(shape[:3], m.stride()[:3])]
        buf = torch.empty(*keep, pad, dtype=dtype, device=device)
        buf[..., :Nk] = m[tuple(slice(0, k) for k in keep)]
        m = buf[..., :Nk].expand(*shape)
    return m


def prefill_workspace_size(q, k, *, rope_cos=None, rope_sin=None, rotary_dim=None) -> int:
    """Workspace bytes ``prefill`` needs (a rotated copy of K for bf16 with
    RoPE, else 0); host-only."""
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if rope_cos is None:
        return 0
    rdim = 2 * rope_cos.shape[1] if rotary_dim is None else int(rotary_dim)
    p = _lib.PrefillParams()
    p.dtype = _dtype_code(q)
    p.batch, p.seqlen_q, p.seqlen_k = B, Nq, Nk
    p.heads_q, p.heads_kv, p.head_dim = Hq, Hkv, d
    p.window_left, p.softmax_scale = -1, 1.0
    p.rotary_dim, p.rope_max_pos = rdim, rope_cos.shape[0]
    st, n = _lib.prefill_workspace_size(p)
    _lib.check(st, "fa_prefill_workspace_size")
    return n


def prefill(q, k, v, *, causal: bool = False, window: int = -1, scale: Optional[float] = None,
            seqlens_q=None, seqlens_k=None, out=None, lse=None, return_lse: bool = True,
            alibi_slopes=None, rope_cos=None, rope_sin=None, rotary_dim=None,
            workspace=None, attn_mask=None) -> Tuple[object, object]:
    """Fused attention forward for a batch of sequences.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] (any strides with a unit last
    stride), bf16 or fp32.  Returns ``(o, lse)`` with o like q ([B, Nq, Hq, d],
    contiguous) and lse fp32 [B, Hq, Nq] (natural log), or ``(o, None)`` when
    ``return_lse`` is False.  ``window`` keeps the last ``window`` keys up to
    and including the diagonal; ``seqlens_q`` / ``seqlens_k`` are per-sequence
    valid lengths (rows past ``seqlens_q`` come back as O = 0, LSE = -inf).
    ``alibi_slopes`` (one value per query head) adds the ALiBi bias
    -slope_h * |pos_i - j| to the scaled scores, pos_i = i + Lk - Lq.
    RoPE: ``rope_cos`` / ``rope_sin`` ([max_pos, rotary_dim / 2] tables;
    ``rotary_dim`` defaults to twice their width) rotate adjacent pairs of the
    first rotary_dim dims of q (at pos_i) and k (at j) before the products.
    bf16 with RoPE needs a workspace (allocated here unless ``workspace``, a
    uint8 GPU tensor of ``prefill_workspace_size`` bytes, is passed).
    ``attn_mask``: an additive mask broadcastable to [B, Hq, Nq, Nk] (for
    example the [B, 1, 1, Nk] key-padding mask), added to the scaled scores;
    -inf removes a key.  It is read in q's dtype; size-1 dims are broadcast
    with stride 0.
    """
    torch = _torch()
    _require_gpu(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, seq, heads, head_dim]")
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"incompatible shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a unit head_dim stride")
    dev = q.device
    if out is None:
        out = torch.empty((B, Nq, Hq, d), dtype=q.dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    sq = _seqlens(seqlens_q, B, dev)
    sk = _seqlens(seqlens_k, B, dev)
    al = _slopes(alibi_slopes, Hq, dev)
    rope = _rope(rope_cos, rope_sin, rotary_dim, dev)
    mask = _mask(attn_mask, q.dtype, (B, Hq, Nq, Nk), dev)
    p = _lib.PrefillParams()
    p.dtype = _dtype_code(q)
    p.batch, p.seqlen_q, p.seqlen_k = B, Nq, Nk
    p.heads_q, p.heads_kv, p.head_dim = Hq, Hkv, d
    p.causal = 1 if causal else 0
    p.window_left = int(window)
    p.softmax_scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    p.q, p.k, p.v, p.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    p.lse = lse.data_ptr() if (return_lse and lse is not None) else None
    p.seqlens_q = sq.data_ptr() if sq is not None else None
    p.seqlens_k = sk.data_ptr() if sk is not None else None
    p.q_stride[:] = [q.stride(0), q.stride(1), q.stride(2)]
    p.k_stride[:] = [k.stride(0), k.stride(1), k.stride(2)]
    p.v_stride[:] = [v.stride(0), v.stride(1), v.stride(2)]
    p.o_stride[:] = [out.stride(0), out.stride(1), out.stride(2)]
    p.alibi_slopes = al.data_ptr() if al is not None else None
    if mask is not None:
        p.attn_mask = mask.data_ptr()
        p.mask_stride[:] = list(mask.stride())
    if rope is not None:
        p.rope_cos, p.rope_sin = rope[0].data_ptr(), rope[1].data_ptr()
        p.rotary_dim, p.rope_max_pos = rope[2], rope[3]
        st, need = _lib.prefill_workspace_size(p)
        _lib.check(st, "fa_prefill_workspace_size")
        if need > 0:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            p.workspace = workspace.data_ptr()
            p.workspace_bytes = workspace.numel() * workspace.element_size()
    _lib.check(_lib.prefill_fwd(p, _stream(dev)), "fa_prefill_fwd")
    return out, (lse if return_lse else None)


def _kv_is_fp8(k_cache, v_cache, k_scale, v_scale) -> bool:
    """FP8 E4M3 caches: torch.float8_e4m3fn tensors, or uint8 codes with scales."""
    torch = _torch()
    fp8 = getattr(torch, "float8_e4m3fn", None)
    kinds = {t.dtype for t in (k_cache, v_cache)}
    if kinds <= {fp8, torch.uint8} and len(kinds) == 1:
        if k_scale is None or v_scale is None:
            raise ValueError("FP8 E4M3 caches need k_scale and v_scale (one per KV head)")
        return True
    if k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale apply to FP8 E4M3 caches only")
    return False


def _kv_scales(x, Hkv, device):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        x = torch.tensor([float(x)] * Hkv if isinstance(x, (int, float)) else list(x),
                         dtype=torch.float32)
    x = x.to(device=device, dtype=torch.float32).contiguous()
    if x.numel() != Hkv:
        raise ValueError(f"k_scale / v_scale must have {Hkv} entries (one per KV head)")
    return x


def _decode_params(q, k_cache, v_cache, sk, out, lse, scale, window, chunk_keys, al=None,
                   table=None, capacity=None, scales=None, rope=None):
    B, Hq, d = q.shape
    _, cap, Hkv, _ = k_cache.shape
    if table is not None:
        # paged: k_cache is the pool [num_pages, page_size, Hkv, d]
        page_size, pages_per_seq = cap, table.shape[1]
        cap = pages_per_seq * page_size if capacity is None else int(capacity)
    p = _lib.DecodeParams()
    p.dtype = _dtype_code(q)
    p.batch, p.heads_q, p.heads_kv, p.head_dim = B, Hq, Hkv, d
    p.cache_capacity = cap
    p.window_left = int(window)
    p.chunk_keys = int(chunk_keys)
    p.softmax_scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    p.reserved0 = 0
    p.q = q.data_ptr()
    p.k_cache, p.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    p.o = out.data_ptr() if out is not None else None
    p.lse = lse.data_ptr() if lse is not None else None
    p.seqlens_k = sk.data_ptr() if sk is not None else None
    p.q_stride[:] = [q.stride(0), q.stride(1)]
    p.k_stride[:] = [k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)]
    p.v_stride[:] = [v_cache.stride(0), v_cache.stride(1), v_cache.stride(2)]
    if out is not None:
        p.o_stride[:] = [out.stride(0), out.stride(1)]
    p.alibi_slopes = al.data_ptr() if al is not None else None
    if table is not None:
        p.block_table = table.data_ptr()
        p.page_size, p.pages_per_seq, p.num_pages = page_size, pages_per_seq, k_cache.shape[0]
    if scales is not None:
        p.kv_format = _lib.FA_KV_FP8_E4M3
        p.k_scale, p.v_scale = scales[0].data_ptr(), scales[1].data_ptr()
    if rope is not None:
        p.rope_cos, p.rope_sin = rope[0].data_ptr(), rope[1].data_ptr()
        p.rotary_dim, p.rope_max_pos = rope[2], rope[3]
    return p


def _block_table(table, B, device):
    torch = _torch()
    if table is None:
        return None
    if not isinstance(table, torch.Tensor):
        table = torch.tensor(table, dtype=torch.int32)
    table = table.to(device=device, dtype=torch.int32).contiguous()
    if table.dim() != 2 or table.shape[0] != B:
        raise ValueError(f"block_table must be [{B}, pages_per_seq]")
    return table


def decode_workspace_size(q, k_cache, v_cache, *, scale=None, window: int = -1,
                          chunk_keys: int = 0, block_table=None, capacity=None,
                          k_scale=None, v_scale=None) -> int:
    """Workspace bytes ``decode`` needs for these shapes (host-only)."""
    table = block_table
    if table is not None and not isinstance(table, _torch().Tensor):
        table = _torch().tensor(table, dtype=_torch().int32)
    # sizing reads shapes only; the table's contents stay where they are
    scales = None
    if _kv_is_fp8(k_cache, v_cache, k_scale, v_scale):
        Hkv = k_cache.shape[2]
        scales = (_kv_scales(k_scale, Hkv, "cpu"), _kv_scales(v_scale, Hkv, "cpu"))
    p = _decode_params(q, k_cache, v_cache, None, None, None, scale, window, chunk_keys,
                       table=table, capacity=capacity, scales=scales)
    st, n = _lib.decode_workspace_size(p)
    _lib.check(st, "fa_decode_workspace_size")
    return n


def decode(q, k_cache, v_cache, seqlens_k, *, scale: Optional[float] = None, window: int = -1,
           chunk_keys: int = 0, workspace=None, out=None, lse=None, return_lse: bool = True,
           alibi_slopes=None, block_table=None, capacity: Optional[int] = None,
           k_scale=None, v_scale=None, rope_cos=None, rope_sin=None, rotary_dim=None):
    """Single-token decode over a KV cache, contiguous or paged.

    q: [B, Hq, d]; k_cache, v_cache: [B, capacity, Hkv, d]; seqlens_k: [B]
    valid lengths (the current token already appended).  Returns ``(o, lse)``:
    o [B, Hq, d] like q, lse fp32 [B, Hq].  ``workspace`` (a uint8 GPU tensor
    of at least ``decode_workspace_size`` bytes) may be passed to avoid an
    allocation per call.  ``alibi_slopes`` (one value per query head) adds the
    ALiBi bias -slope_h * (L_b - 1 - j).

    Paged cache: with ``block_table`` (int32 [B, pages_per_seq]) the caches are
    page pools [num_pages, page_size, Hkv, d]; logical row j of sequence b is
    row j % page_size of page block_table[b, j // page_size].  ``capacity``
    (default pages_per_seq * page_size) caps the lengths.

    FP8 cache: caches of dtype ``torch.float8_e4m3fn`` (or ``uint8`` codes)
    hold OCP FP8 E4M3 values; ``k_scale`` and ``v_scale`` (one fp32 value per
    KV head, or one float for all) give element = scale * E4M3(code).  q and
    the output stay bf16.

    RoPE: ``rope_cos`` / ``rope_sin`` tables ([max_pos, rotary_dim / 2])
    rotate the query at its position L_b - 1; cached keys are used as stored
    (already rotated when they were appended).
    """
    torch = _torch()
    _require_gpu(q, k_cache, v_cache)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, Hq, d] and caches [B, capacity, Hkv, d] "
                         "(or pools [num_pages, page_size, Hkv, d])")
    B, Hq, d = q.shape
    table = _block_table(block_table, B, q.device)
    if (table is None and k_cache.shape[0] != B) or k_cache.shape[3] != d:
        raise ValueError("cache shape does not match q")
    fp8 = _kv_is_fp8(k_cache, v_cache, k_scale, v_scale)
    if not fp8 and not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share one dtype")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name} must have a unit head_dim stride")
    dev = q.device
    sk = _seqlens(seqlens_k, B, dev)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=q.dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    al = _slopes(alibi_slopes, Hq, dev)
    scales = None
    if fp8:
        Hkv = k_cache.shape[2]
        scales = (_kv_scales(k_scale, Hkv, dev), _kv_scales(v_scale, Hkv, dev))
    rope = _rope(rope_cos, rope_sin, rotary_dim, dev)
    p = _decode_params(q, k_cache, v_cache, sk, out, lse if return_lse else None, scale, window,
                       chunk_keys, al, table, capacity, scales, rope)
    if isinstance(workspace, str) and workspace == "noalloc":
        _lib.check(_lib.decode_fwd_noalloc(p, _stream(dev)), "fa_decode_fwd_noalloc")
        return out, (lse if return_lse else None)
    st, need = _lib.decode_workspace_size(p)
    _lib.check(st, "fa_decode_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _lib.check(_lib.decode_fwd(p, workspace.data_ptr(), ws_bytes, _stream(dev)), "fa_decode_fwd")
    return out, (lse if return_lse else None)


def decode_noalloc(q, k_cache, v_cache, seqlens_k, *, out, lse=None, **kw):
    """``decode`` through fa_decode_fwd_noalloc: the partial results live in
    the library's own device array, so with ``out`` (and ``lse``, or
    ``return_lse=False``) preallocated, and device tensors for the lengths
    (and slopes, scales, tables), the call allocates nothing.  Calls that
    overlap in time on one GPU share that array and race; calls ordered on
    one stream are safe.  Problems whose workspace would exceed
    ``DECODE_NOALLOC_MAX_BYTES`` raise FAError (FA_ERR_WORKSPACE)."""
    if kw.get("return_lse", True) and lse is None:
        raise ValueError("decode_noalloc needs a preallocated lse (or return_lse=False)")
    return decode(q, k_cache, v_cache, seqlens_k, out=out, lse=lse, workspace="noalloc", **kw)
