"""GPU parity: the explicit additive mask (attn_mask) of fa_prefill_fwd
against the fp64 oracle, which adds the same stored values to the scaled
scores.  Masks are drawn here (seeded), stored in the call's dtype, and
passed with broadcast strides where their shape has size-1 dims.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import DEV, check, prefill_inputs, say, to_np

pytestmark = pytest.mark.gpu


def _stored(m, dtype):
    """The mask as stored (bf16 bits, half bits or fp32) and its exact float64 values."""
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(m.astype(np.float32))
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        return t, workloads.bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "f16":
        h = np.ascontiguousarray(m, dtype=np.float32).astype(np.float16)
        return torch.from_numpy(h), h.astype(np.float64)
    f = m.astype(np.float32)
    return torch.from_numpy(f), f.astype(np.float64)


def _case(p, mask, ctx, **kw):
    say(f"[mask] {ctx} shape={p.shape} {p.dtype} causal={p.causal} W={p.window_left} "
        f"mask={mask.shape}")
    mt, mv = _stored(mask, p.dtype)
    q, k, v, sq, sk = prefill_inputs(p)
    o, lse = fa.prefill(q, k, v, causal=p.causal, window=p.window_left, scale=p.scale,
                        seqlens_q=sq, seqlens_k=sk, attn_mask=mt.to(DEV), **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(workloads.to_f64(p.q, p.dtype), workloads.to_f64(p.k, p.dtype),
                              workloads.to_f64(p.v, p.dtype), scale=p.scale, causal=p.causal,
                              window_left=p.window_left, seqlens_q=p.seqlens_q,
                              seqlens_k=p.seqlens_k, attn_mask=mv,
                              alibi_slopes=kw.get("alibi_slopes"))
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, p.dtype, ctx)


def test_key_padding_mask_bert_layout():
    """The BERT page's [b, 1, 1, n] mask: 0 on real keys, -inf past each length."""
    p = workloads.make_prefill(120, 4, 512, 512, 12, 12, 64, "bf16")
    lengths = [512, 300, 129, 1]
    m = np.zeros((4, 1, 1, 512))
    for b, L in enumerate(lengths):
        m[b, 0, 0, L:] = -np.inf
    _case(p, m, "BERT key padding")


def test_large_negative_padding_values():
    # masks in practice often hold a large finite negative instead of -inf
    p = workloads.make_prefill(121, 2, 256, 256, 4, 4, 128, "bf16", causal=True)
    m = np.zeros((2, 1, 1, 256))
    m[0, 0, 0, 200:] = -10000.0
    _case(p, m, "padding as -1e4")


@pytest.mark.parametrize("shape", [(2, 8, 300, 333), (2, 1, 300, 333), (1, 8, 300, 333),
                                   (300, 333)])
def test_dense_random_mask_broadcasts(shape):
    """A dense random bias (some -inf) over GQA causal attention with ragged
    key count (the last 8-key run of a row is partial)."""
    p = workloads.make_prefill(122, 2, 300, 333, 8, 2, 128, "bf16", causal=True)
    rng = np.random.default_rng(123)
    m = rng.standard_normal(shape) * 2.0
    m[rng.random(shape) < 0.05] = -np.inf
    _case(p, m, f"dense mask {shape}")


# Key masks (one row per batch and head, broadcast over the query rows: row
# stride 0) take the matrix-core path: the mask value enters the scores as one
# more k-step of the S product.

@pytest.mark.parametrize("dtype,d,Hq,Hkv", [("bf16", 128, 8, 2), ("bf16", 64, 4, 4),
                                             ("f16", 128, 4, 1), ("f16", 64, 6, 3)])
def test_key_mask_per_head_random(dtype, d, Hq, Hkv):
    """Random key-mask rows per batch and head (some -inf), causal, a ragged
    key count, GQA (packed for bf16 d128), valid key lengths."""
    p = workloads.make_prefill(130, 2, 300, 333, Hq, Hkv, d, dtype, causal=True,
                               seqlens_k_range=(200, 333))
    rng = np.random.default_rng(131)
    m = rng.standard_normal((2, Hq, 1, 333)) * 3.0
    m[rng.random(m.shape) < 0.1] = -np.inf
    _case(p, m, f"key mask [2,{Hq},1,333] {dtype} d{d}")


def test_key_mask_with_alibi_window():
    p = workloads.make_prefill(132, 2, 400, 400, 4, 2, 128, "bf16", causal=True, window_left=150)
    rng = np.random.default_rng(133)
    m = rng.standard_normal((2, 1, 1, 400)) * 2.0
    m[:, :, :, 390:] = -np.inf
    _case(p, m, "key mask + ALiBi + window",
          alibi_slopes=np.array([0.02, 0.05, 0.1, 0.2], dtype=np.float32))


def test_key_mask_large_and_tiny_values():
    """Magnitudes far from 1 (the mask times 1/scale must keep fp32 accuracy):
    -1e4 on some keys (masking them), +-30 on others (they dominate their
    rows), +-1e-3 on the rest; non-causal, d128.  (A row dominated by a
    +1e4 key would have an LSE near 1e4, where fp32 spacing alone is about
    1e-3, the LSE bound.)"""
    p = workloads.make_prefill(134, 1, 257, 257, 2, 2, 128, "bf16")
    rng = np.random.default_rng(135)
    m = rng.standard_normal((1, 2, 1, 257)) * 1e-3
    u = rng.random(m.shape)
    m[u < 0.3] = -1e4
    mid = u > 0.9
    m[mid] = np.sign(rng.standard_normal(int(mid.sum()))) * 30.0
    _case(p, m, "key mask of -1e4, +-30 and +-1e-3")


def test_key_mask_non_default_scale():
    """A softmax scale whose inverse is a 16-bit value (so two of the three
    parts of 1/scale are zero) and one that needs all three, with -inf keys."""
    for scale in (0.25, 0.0917):
        p = workloads.make_prefill(136, 1, 200, 200, 2, 2, 128, "bf16", causal=True, scale=scale)
        m = np.zeros((1, 1, 1, 200))
        m[0, 0, 0, 150:] = -np.inf
        m[0, 0, 0, :20] = 1.5
        _case(p, m, f"key mask, scale {scale}")


def test_mask_that_removes_whole_rows():
    p = workloads.make_prefill(124, 1, 130, 130, 2, 2, 128, "bf16")
    m = np.zeros((1, 2, 130, 130))
    m[0, 0, 5] = -np.inf                      # row 5 of head 0 sees nothing
    m[0, 1, :, 64:] = -np.inf                 # head 1 sees only the first tile
    _case(p, m, "rows removed by the mask")


def test_mask_with_alibi_window_and_d64():
    p = workloads.make_prefill(125, 2, 400, 400, 4, 2, 64, "bf16", causal=True, window_left=150)
    m = np.random.default_rng(126).standard_normal((2, 4, 400, 400))
    _case(p, m, "mask + ALiBi + window, d64",
          alibi_slopes=np.array([0.02, 0.05, 0.1, 0.2], dtype=np.float32))


@pytest.mark.parametrize("kw", [dict(causal=True), dict()])
def test_mask_fp32(kw):
    p = workloads.make_prefill(127, 2, 150, 170, 2, 1, 64, "f32", **kw)
    m = np.random.default_rng(128).standard_normal((2, 1, 150, 170))
    m[:, :, :, 160:] = -np.inf
    _case(p, m, f"fp32 mask {kw}")


def test_mask_8k_key_padding_sampled():
    """The causal N=8192 workload under a key-padding mask, sampled rows."""
    p = workloads.make_workload(3)
    m = np.zeros((1, 1, 1, 8192))
    m[0, 0, 0, 6000:] = -np.inf
    mt, mv = _stored(m, "bf16")
    q, k, v, sq, sk = prefill_inputs(p)
    say("[mask] 8k causal with key padding at 6000, sampled rows")
    o, lse = fa.prefill(q, k, v, causal=True, scale=p.scale, attn_mask=mt.to(DEV))
    torch.cuda.synchronize()
    rows = np.array([0, 5999, 6000, 6001, 8191])
    heads = np.array([0, 31])
    ro, rl = oracle.attention(workloads.to_f64(p.q, "bf16"), workloads.to_f64(p.k, "bf16"),
                              workloads.to_f64(p.v, "bf16"), scale=p.scale, causal=True,
                              rows=rows, heads=heads, attn_mask=mv)
    check(to_np(o)[:, rows][:, :, heads], lse.cpu().numpy().astype(np.float64)[:, heads][:, :, rows],
          ro, rl, "bf16", "8k key padding")
