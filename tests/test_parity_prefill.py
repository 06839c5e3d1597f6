"""GPU parity: fa_prefill_fwd (through the C ABI) against the fp64 oracle.

Small and medium problems are compared element by element on all outputs;
the two full-size causal workloads (N = 8192 and the GQA window workload) are
compared on sampled rows and heads, which the oracle computes one by one.
Every case prints its name and shape before the GPU call.
"""
import numpy as np
import pytest
import torch

import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import DEV, check, dev_tensor, oracle_prefill, prefill_inputs, run_prefill, say

pytestmark = pytest.mark.gpu


def _case(p, ctx):
    say(f"[prefill] {ctx} shape(B,Nq,Nk,Hq,Hkv,d)={p.shape} dtype={p.dtype} causal={p.causal} "
        f"W={p.window_left} seqlens_q={p.seqlens_q is not None} seqlens_k={p.seqlens_k is not None}")
    o, lse = run_prefill(p)
    ro, rl = oracle_prefill(p)
    check(o, lse, ro, rl, p.dtype, ctx)
    return o, lse


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------
def test_workload1_tiny_fp32():
    _case(workloads.make_workload(1), "tiny fp32 B1 H1 N128 d64")


def test_workload2_bert_varlen():
    _case(workloads.make_workload(2), "BERT-base B8 H12 N512 d64 key lengths U[128,512]")


def _sampled(p, ctx, rows, heads):
    say(f"[prefill] {ctx} (full size, sampled rows) shape={p.shape}")
    o, lse = run_prefill(p)
    assert np.all(np.isfinite(o)), "non-finite output"
    ro, rl = oracle_prefill(p, rows=rows, heads=heads)
    check(o[:, rows][:, :, heads], lse[:, heads][:, :, rows], ro, rl, p.dtype, ctx)


def test_workload3_causal_8k_sampled():
    p = workloads.make_workload(3)
    rng = np.random.default_rng(303)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 129, 4095, 4096, 8190, 8191],
                                     rng.integers(0, 8192, 40)]))
    heads = np.array([0, 5, 17, 31])
    _sampled(p, "decoder-7B causal B1 H32 N8192 d128", rows, heads)


def test_workload4_gqa_window_sampled():
    p = workloads.make_workload(4)
    rng = np.random.default_rng(404)
    rows = np.unique(np.concatenate([[0, 1, 1023, 1024, 1025, 2047, 2048, 4095],
                                     rng.integers(0, 4096, 40)]))
    heads = np.array([0, 3, 4, 13, 31])
    _sampled(p, "GQA causal window-1024 B2 Hq32 Hkv8 N4096 d128", rows, heads)


# ---------------------------------------------------------------------------
# Scaled-down versions of the full-size workloads, compared on every output
# ---------------------------------------------------------------------------
def test_causal_mha_medium_all_rows():
    _case(workloads.make_prefill(33, 1, 1100, 1100, 4, 4, 128, "bf16", causal=True),
          "causal MHA N1100 d128")


def test_gqa_window_medium_all_rows():
    _case(workloads.make_prefill(44, 2, 1000, 1000, 8, 2, 128, "bf16", causal=True,
                                 window_left=256), "causal GQA window256 N1000 d128")


# ---------------------------------------------------------------------------
# Edge cases: ragged extents, windows, MQA, valid lengths, fp32 variants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N", [1, 2, 17, 63, 65, 127, 129, 255, 509])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(N, causal):
    _case(workloads.make_prefill(100 + N, 2, N, N, 4, 2, 128, "bf16", causal=causal),
          f"ragged N{N} causal={causal}")


@pytest.mark.parametrize("N", [1, 2, 15, 16, 17, 127, 129, 143])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_ragged_lengths(N, causal, d):
    """The fp32 kernel's eight wavefronts take alternate 16-key tiles: below
    eight tiles some wavefronts merge an empty partial (max -inf, sum 0), and
    the last tile is ragged.  MQA (one KV head)."""
    _case(workloads.make_prefill(300 + N + d, 2, N, N, 2, 1, d, "f32", causal=causal),
          f"fp32 ragged N{N} d{d} causal={causal}")


@pytest.mark.parametrize("W", [1, 63, 64, 65, 200, 700])
def test_causal_windows(W):
    _case(workloads.make_prefill(200 + W, 1, 600, 600, 4, 2, 128, "bf16", causal=True,
                                 window_left=W), f"causal window {W}")


def test_window_without_causal():
    _case(workloads.make_prefill(7, 2, 300, 300, 2, 2, 64, "bf16", window_left=100),
          "window 100, not causal")


def test_mqa_single_kv_head():
    _case(workloads.make_prefill(8, 2, 257, 257, 8, 1, 128, "bf16", causal=True), "MQA Hkv=1")


def test_head_dim_64_noncausal_gqa():
    _case(workloads.make_prefill(9, 3, 333, 333, 6, 3, 64, "bf16"), "d64 GQA non-causal")


def test_key_lengths_with_empty_and_single():
    p = workloads.make_prefill(10, 4, 300, 300, 4, 4, 128, "bf16")
    p.seqlens_k = np.array([0, 1, 77, 300], dtype=np.int32)
    _case(p, "key lengths 0,1,77,300")


def test_query_and_key_lengths():
    p = workloads.make_prefill(11, 3, 400, 400, 4, 2, 128, "bf16", causal=True,
                               seqlens_k_range=(1, 400), seqlens_q_equal_k=True)
    _case(p, "q and k valid lengths, causal")


def test_causal_fewer_keys_than_queries():
    # bottom-right alignment: the first Lq - Lk rows see nothing
    p = workloads.make_prefill(12, 2, 300, 300, 2, 2, 128, "bf16", causal=True)
    p.seqlens_k = np.array([100, 299], dtype=np.int32)
    _case(p, "causal with Lk < Lq")


@pytest.mark.parametrize("Nq,Nk", [(100, 333), (333, 100), (64, 1000)])
@pytest.mark.parametrize("causal", [False, True])
def test_cross_lengths(Nq, Nk, causal):
    _case(workloads.make_prefill(13 + Nq, 2, Nq, Nk, 4, 2, 128, "bf16", causal=causal),
          f"Nq{Nq} Nk{Nk} causal={causal}")


@pytest.mark.parametrize("kw", [dict(causal=True), dict(causal=True, window_left=37),
                                dict(seqlens_k_range=(1, 200)), dict()])
def test_fp32_variants(kw):
    _case(workloads.make_prefill(14, 2, 200, 200, 4, 2, 128, "f32", **kw), f"fp32 {kw}")
    _case(workloads.make_prefill(15, 1, 130, 130, 2, 1, 64, "f32", **kw), f"fp32 d64 {kw}")


def test_large_score_offset_is_stable():
    """K -> K + u makes raw scores ~ +-100s; max subtraction keeps exp finite."""
    p = workloads.make_prefill(16, 1, 300, 300, 2, 2, 128, "bf16", causal=True)
    k = workloads.bf16_bits_to_f32(p.k) + np.float32(8.0)
    p.k = workloads.f32_to_bf16_bits(k)
    q = workloads.bf16_bits_to_f32(p.q) + np.float32(4.0)
    p.q = workloads.f32_to_bf16_bits(q)
    _case(p, "large score offsets")


def _growing_scores(p, rate):
    """Rewrite Q and K so that, for even query rows, scale*q.k grows by about
    `rate` (base-2 exponent units) per 64 keys along the key axis, and falls as
    fast for odd rows: rows of one wavefront then move their softmax
    reference at different tiles."""
    B, Nq, Hq, d = p.q.shape
    Nk, Hkv = p.k.shape[1], p.k.shape[2]
    q = 0.1 * workloads.bf16_bits_to_f32(p.q).astype(np.float64)
    k = 0.1 * workloads.bf16_bits_to_f32(p.k).astype(np.float64)
    sign = np.where(np.arange(Nq) % 2 == 0, 1.0, -1.0)[None, :, None, None]
    q += sign
    # scale*log2(e)*d*g per key; g grows linearly with the key index
    g = rate * np.arange(Nk) / 64.0 / (p.scale * np.log2(np.e) * d)
    k += g[None, :, None, None]
    p.q = workloads.f32_to_bf16_bits(q.astype(np.float32))
    p.k = workloads.f32_to_bf16_bits(k.astype(np.float32))
    return p


@pytest.mark.parametrize("causal", [True, False])
def test_reference_moves_under_growing_scores(causal):
    """Scores that grow (or fall) by ~20 base-2 units per tile force the softmax
    reference of half the rows of every wavefront to move on most tiles."""
    p = _growing_scores(workloads.make_prefill(21, 1, 1000, 1000, 2, 2, 128, "bf16",
                                               causal=causal), 20.0)
    _case(p, f"growing scores causal={causal}")


# ---------------------------------------------------------------------------
# Padding, poisoning, canaries, determinism, layouts, memory
# ---------------------------------------------------------------------------
def test_poisoned_padding_matches_unpadded_prefix():
    p = workloads.make_prefill(17, 3, 300, 300, 4, 2, 128, "bf16", causal=True,
                               seqlens_k_range=(1, 300), seqlens_q_equal_k=True,
                               poison_padding=True)
    o, lse = _case(p, "NaN-poisoned padding")
    for b in range(3):
        L = int(p.seqlens_k[b])
        sub = workloads.PrefillProblem("bf16", p.q[b:b + 1, :L].copy(), p.k[b:b + 1, :L].copy(),
                                       p.v[b:b + 1, :L].copy(), p.scale, True)
        o2, l2 = run_prefill(sub)
        # same kernel, same tiles over the valid prefix: identical bits
        assert np.array_equal(o[b:b + 1, :L], o2)
        assert np.array_equal(lse[b:b + 1, :, :L], l2)


def test_no_writes_outside_outputs():
    p = workloads.make_prefill(18, 2, 130, 130, 4, 2, 128, "bf16", causal=True)
    q, k, v, _, _ = prefill_inputs(p)
    n_o = q.numel()
    pad = 4096
    o_buf = torch.full((n_o + 2 * pad,), 512.0, dtype=torch.bfloat16, device=DEV)
    l_buf = torch.full((2 * 4 * 130 + 2 * pad,), 777.0, dtype=torch.float32, device=DEV)
    o = o_buf[pad:pad + n_o].view(q.shape)
    lse = l_buf[pad:pad + 2 * 4 * 130].view(2, 4, 130)
    fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o_buf[:pad] == 512.0) and torch.all(o_buf[pad + n_o:] == 512.0)
    assert torch.all(l_buf[:pad] == 777.0) and torch.all(l_buf[pad + 2 * 4 * 130:] == 777.0)
    ro, rl = oracle_prefill(p)
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
          ro, rl, "bf16", "canaries")


def test_run_to_run_bit_identical():
    p = workloads.make_prefill(19, 2, 700, 700, 8, 2, 128, "bf16", causal=True, window_left=300)
    q, k, v, _, _ = prefill_inputs(p)
    outs = [fa.prefill(q, k, v, causal=True, window=300, scale=p.scale) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_strided_layouts_bhsd_and_packed_qkv():
    p = workloads.make_prefill(20, 2, 200, 200, 4, 4, 128, "bf16", causal=True)
    ro, rl = oracle_prefill(p)
    q, k, v, _, _ = prefill_inputs(p)
    # BHSD storage viewed as BSHD
    qb, kb, vb = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    o, lse = fa.prefill(qb, kb, vb, causal=True, scale=p.scale)
    torch.cuda.synchronize()
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
          ro, rl, "bf16", "BHSD strides")
    # one packed [B, N, 3, H, d] buffer
    qkv = torch.stack([q, k, v], dim=2).contiguous()
    o2, lse2 = fa.prefill(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], causal=True, scale=p.scale)
    torch.cuda.synchronize()
    check(o2.float().cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64),
          ro, rl, "bf16", "packed QKV")


def test_no_device_allocation_and_optional_lse():
    p = workloads.make_prefill(21, 1, 512, 512, 4, 4, 128, "bf16", causal=True)
    q, k, v, _, _ = prefill_inputs(p)
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 512), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(DEV) == before
    o2, none = fa.prefill(q, k, v, causal=True, scale=p.scale, return_lse=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))


def test_rejects_cpu_tensors():
    p = workloads.make_prefill(22, 1, 8, 8, 1, 1, 64, "f32")
    t = torch.from_numpy(p.q)
    with pytest.raises(ValueError):
        fa.prefill(t, t, t)


# ---------------------------------------------------------------------------
# ALiBi bias (-m_h |pos_i - j| added to the scaled scores)
# ---------------------------------------------------------------------------
def _slopes(H, base=8.0):
    # a geometric sequence of slopes, one per head (any values are valid inputs)
    return [2.0 ** (-base * (h + 1) / H) for h in range(H)]


def _alibi_case(p, slopes, ctx):
    say(f"[prefill] {ctx} shape(B,Nq,Nk,Hq,Hkv,d)={p.q.shape[0], p.q.shape[1], p.k.shape[1], p.q.shape[2], p.k.shape[2], p.q.shape[3]} "
        f"causal={p.causal} W={p.window_left} slopes={['%.3g' % s for s in slopes]}")
    o, lse = run_prefill(p, alibi_slopes=slopes)
    ro, rl = oracle_prefill(p, alibi_slopes=slopes)
    check(o, lse, ro, rl, p.dtype, ctx)


@pytest.mark.parametrize("causal", [True, False])
def test_alibi_mha_all_rows(causal):
    p = workloads.make_prefill(60, 1, 700, 700, 4, 4, 128, "bf16", causal=causal)
    _alibi_case(p, _slopes(4), f"ALiBi causal={causal}")


def test_alibi_gqa_window_lengths_and_offset():
    """GQA, sliding window and valid lengths with Lq < Lk, so every query's
    position is shifted by Lk - Lq in both the mask and the bias."""
    p = workloads.make_prefill(61, 3, 300, 420, 8, 2, 128, "bf16", causal=True, window_left=150)
    p.seqlens_q = np.array([300, 120, 1], dtype=np.int32)
    p.seqlens_k = np.array([420, 400, 77], dtype=np.int32)
    _alibi_case(p, _slopes(8, 4.0), "ALiBi GQA window Lq<Lk")


def test_alibi_head_dim_64_and_fp32():
    _alibi_case(workloads.make_prefill(62, 2, 333, 333, 6, 3, 64, "bf16"), _slopes(6),
                "ALiBi d64 non-causal")
    _alibi_case(workloads.make_prefill(63, 2, 200, 200, 4, 2, 128, "f32", causal=True),
                _slopes(4), "ALiBi fp32 causal")


def test_alibi_large_slopes_and_zero_slopes():
    """Huge slopes concentrate every row on its own key position (O -> V_pos);
    zero slopes give the plain result (to rounding only: the ALiBi kernel
    visits the key tiles last to first, so its sums run in another order)."""
    p = workloads.make_prefill(64, 1, 260, 260, 2, 2, 128, "bf16", causal=True)
    _alibi_case(p, [50.0, 200.0], "ALiBi huge slopes")
    _alibi_case(p, [0.0, 0.0], "ALiBi zero slopes")
    q, k, v, sq, sk = prefill_inputs(p)
    o0, l0 = fa.prefill(q, k, v, causal=True, scale=p.scale)
    o1, l1 = fa.prefill(q, k, v, causal=True, scale=p.scale, alibi_slopes=[0.0, 0.0])
    torch.cuda.synchronize()
    assert (o0.float() - o1.float()).abs().max().item() <= 2e-2
    assert (l0 - l1).abs().max().item() <= 1e-5


def test_alibi_causal_8k_sampled():
    """Full-size causal N=8192 with ALiBi, sampled rows and heads."""
    p = workloads.make_workload(3)
    slopes = _slopes(p.q.shape[2])
    rows = np.array([0, 1, 63, 64, 255, 256, 4095, 4096, 8000, 8191])
    heads = np.array([0, 7, 31])
    say(f"[prefill] ALiBi causal 8k sampled rows={rows.tolist()} heads={heads.tolist()}")
    o, lse = run_prefill(p, alibi_slopes=slopes)
    ro, rl = oracle_prefill(p, rows=rows, heads=heads, alibi_slopes=slopes)
    check(o[:, rows][:, :, heads], lse[:, heads][:, :, rows], ro, rl, p.dtype, "ALiBi 8k sampled")


def test_long_sequence_sampled_rows():
    """N = 40000 (not a tile multiple) on one head: long key ranges and large
    row indices, sampled rows against the oracle."""
    p = workloads.make_prefill(160, 1, 40000, 40000, 1, 1, 128, "bf16", causal=True)
    rows = np.array([0, 1, 255, 256, 20000, 39743, 39744, 39998, 39999])
    _sampled(p, "causal N40000 H1", rows, np.array([0]))


def test_batch_offsets_beyond_2_31_elements():
    """Maximum sizes: a padded extent of 3 x 131072 rows x 64 heads x 128 dims
    (6 GiB per bf16 tensor), so the third sequence starts 2^31 elements (4 GiB)
    into Q, K, V and O.  The valid prefixes (seeded, at most 512 rows) sit at
    the start of each sequence and everything else is NaN; the padded query
    rows must come back O = 0, LSE = -inf, and the valid ones match the oracle
    on the same values."""
    B, N, H, d = 3, 131072, 64, 128
    p = workloads.make_prefill(190, B, 512, 512, H, H, d, "bf16", causal=True,
                               seqlens_k_range=(100, 512), seqlens_q_equal_k=True,
                               poison_padding=True)
    say(f"[prefill] offsets past 2^31 elements: B={B} N={N} H={H} lengths={list(p.seqlens_k)}")
    q, k, v = (torch.full((B, N, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
               for _ in range(3))
    for big, small in zip((q, k, v), (p.q, p.k, p.v)):
        big[:, :512] = dev_tensor(small, "bf16")
    assert q[2].data_ptr() - q.data_ptr() == 2 ** 31 * 2
    sl = torch.from_numpy(p.seqlens_k).to(DEV)
    o, lse = fa.prefill(q, k, v, causal=True, scale=p.scale, seqlens_q=sl, seqlens_k=sl)
    torch.cuda.synchronize()
    del q, k, v
    assert int(o[:, 512:].abs().amax()) == 0, "padded rows beyond the drawn prefix not zero"
    assert bool(torch.all(lse[:, :, 512:] == float("-inf")))
    heads = [0, 31, 63]
    ro, rl = oracle_prefill(p, heads=heads)
    check(to_np_rows(o[:, :512, heads]), lse[:, heads, :512].cpu().numpy().astype(np.float64),
          ro, rl, "bf16", "offsets past 2^31 elements")
    del o, lse
    torch.cuda.empty_cache()


def to_np_rows(t):
    return t.float().cpu().numpy().astype(np.float64)
