"""GPU parity: fa_decode_fwd (split-KV decode + LSE combine, through the C
ABI) against the fp64 oracle.  Caches come from the generator with every row
at or beyond a sequence's length set to NaN, so any read past the valid
prefix would poison the output.
"""
import numpy as np
import pytest
import torch

import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import (DEV, check, decode_inputs, dev_tensor, oracle_decode, run_decode, say,
                         to_np)

pytestmark = pytest.mark.gpu


def _case(dp, ctx, **kw):
    say(f"[decode] {ctx} B={dp.q.shape[0]} Hq={dp.q.shape[1]} Hkv={dp.k_cache.shape[2]} "
        f"d={dp.q.shape[2]} cap={dp.k_cache.shape[1]} W={dp.window_left} {kw}")
    o, lse = run_decode(dp, **kw)
    ro, rl = oracle_decode(dp)
    check(o, lse, ro, rl, dp.dtype, ctx)
    return o, lse


def test_workload5_decode_full():
    _case(workloads.make_workload(5), "decode B64 Hq32 Hkv8 d128 L U[512,8192]")


@pytest.mark.parametrize("chunk", [0, 128, 256, 512])
def test_lengths_around_chunk_edges(chunk):
    # edges of the 32-key tiles, the 128-key tile rounds of a workgroup and the chunks
    lengths = np.array([1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384,
                        385, 511, 512, 513, 600, 0, 1000], dtype=np.int32)
    dp = workloads.make_decode(50, len(lengths), 8, 2, 128, 1000, (1, 1000), "bf16",
                               lengths=lengths)
    _case(dp, f"lengths at chunk edges, chunk={chunk}", chunk_keys=chunk)


@pytest.mark.parametrize("chunk", [0, 128, 384])
def test_many_sequences_work_order(chunk):
    # more than one block of 64 sequences (the split kernel orders each
    # block's work items longest chunk first): repeated lengths (ties),
    # empty sequences, and sequences that fill the capacity
    rng = np.random.default_rng(70)
    lengths = rng.integers(1, 700, size=150).astype(np.int32)
    lengths[[3, 64, 65, 127, 128, 149]] = 0
    lengths[[10, 20, 70, 140]] = 700
    lengths[30:40] = 257
    dp = workloads.make_decode(71, len(lengths), 8, 2, 128, 700, (1, 700), "bf16",
                               lengths=lengths)
    o, lse = _case(dp, f"150 sequences, chunk={chunk}", chunk_keys=chunk)
    # no atomics and a fixed order: the same call again is bit-identical
    o2, lse2 = run_decode(dp, chunk_keys=chunk)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_large_batch_item_table():
    """Batches above 64 sequences take their work items from the table a
    one-workgroup plan kernel writes (16 blocks of 64 per round): 1100
    sequences (two rounds, a partial block) with empty, full and tied
    lengths, compared on every sequence; the same call again is
    bit-identical; a paged and an FP8 cache of 300 sequences go the same
    way."""
    rng = np.random.default_rng(72)
    lengths = rng.integers(0, 300, size=1100).astype(np.int32)
    lengths[::97] = 0
    lengths[5::101] = 300
    lengths[200:260] = 129
    dp = workloads.make_decode(73, len(lengths), 4, 2, 64, 300, (0, 300), "bf16",
                               lengths=lengths)
    o, lse = _case(dp, "1100 sequences (item table)", chunk_keys=128)
    o2, lse2 = run_decode(dp, chunk_keys=128)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    from gpu_helpers import oracle_decode_paged, run_decode_fp8, run_decode_paged
    pp = workloads.make_decode_paged(74, 300, 8, 2, 128, 512, (0, 512), 32, "bf16")
    say("[decode] 300 sequences, paged pool of 32-row pages (item table)")
    o, lse = run_decode_paged(pp)
    ro, rl = oracle_decode_paged(pp)
    check(o, lse, ro, rl, "bf16", "300 sequences paged")
    from gpu_helpers import oracle_decode_fp8
    df = workloads.make_decode(75, 300, 8, 2, 128, 512, (0, 512), "bf16", kv_dtype="fp8_e4m3")
    say("[decode] 300 sequences, FP8 cache (item table)")
    o, lse = run_decode_fp8(df)
    ro, rl = oracle_decode_fp8(df)
    check(o, lse, ro, rl, "bf16", "300 sequences FP8")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (16, 4), (32, 4), (6, 2), (8, 1), (12, 4)])
def test_gqa_groups(Hq, Hkv):
    dp = workloads.make_decode(51 + Hq, 5, Hq, Hkv, 128, 900, (1, 900), "bf16")
    _case(dp, f"GQA Hq{Hq} Hkv{Hkv}")


@pytest.mark.parametrize("chunk", [0, 128, 512])
def test_head_dim_64(chunk):
    dp = workloads.make_decode(52, 6, 12, 4, 64, 777, (1, 777), "bf16")
    _case(dp, "d64", chunk_keys=chunk)


@pytest.mark.parametrize("W", [1, 64, 100, 5000])
def test_window(W):
    dp = workloads.make_decode(53, 6, 8, 2, 128, 1200, (1, 1200), "bf16", window_left=W)
    _case(dp, f"window {W}")


def test_lengths_clamped_to_capacity():
    # every cache row valid, so lengths beyond capacity clamp onto real data
    dp = workloads.make_decode(54, 3, 4, 2, 128, 300, (1, 300), "bf16",
                               lengths=np.array([300, 300, 300], dtype=np.int32))
    q, kc, vc, sk = decode_inputs(dp)
    big = torch.tensor([5000, -7, 300], dtype=torch.int32, device=DEV)
    o, lse = fa.decode(q, kc, vc, big, scale=dp.scale)
    torch.cuda.synchronize()
    # reference with the clamped lengths; the oracle clamps the same way
    dp.seqlens_k = np.array([5000, -7, 300], dtype=np.int32)
    ro, rl = oracle_decode(dp)
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", "clamped lengths")


def test_reference_moves_under_growing_scores():
    """Keys whose scores grow by ~20 base-2 units per 32 keys force the running
    reference of every wavefront to move on most tiles (and every chunk's
    partial to sit at a very different max, which the combine must merge)."""
    dp = workloads.make_decode(57, 4, 8, 2, 128, 1500, (600, 1500), "bf16")
    q = 0.1 * workloads.bf16_bits_to_f32(dp.q).astype(np.float64) + 1.0
    k = workloads.bf16_bits_to_f32(dp.k_cache).astype(np.float64)
    cap = k.shape[1]
    g = 20.0 * np.arange(cap) / 32.0 / (dp.scale * np.log2(np.e) * 128)
    k = np.where(np.isnan(k), k, 0.1 * k + g[None, :, None, None])
    dp.q = workloads.f32_to_bf16_bits(q.astype(np.float32))
    dp.k_cache = workloads.f32_to_bf16_bits(k.astype(np.float32))
    _case(dp, "growing scores")


def test_chunk_sizes_agree():
    dp = workloads.make_decode(55, 8, 8, 2, 128, 2000, (1, 2000), "bf16")
    outs = [run_decode(dp, chunk_keys=c) for c in (128, 256, 512, 1024)]
    for o, l in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= 2e-2
        assert np.abs(l - outs[0][1]).max() <= 1e-3


def test_decode_equals_single_query_prefill():
    """The decode query is a one-row bottom-right-aligned causal prefill."""
    dp = workloads.make_decode(56, 5, 8, 2, 128, 520, (1, 520), "bf16")
    q, kc, vc, sk = decode_inputs(dp)
    od, ld = fa.decode(q, kc, vc, sk, scale=dp.scale)
    op, lp = fa.prefill(q[:, None], kc, vc, causal=True, scale=dp.scale,
                        seqlens_q=torch.ones(5, dtype=torch.int32, device=DEV), seqlens_k=sk)
    torch.cuda.synchronize()
    assert np.abs(to_np(od) - to_np(op[:, 0])).max() <= 2e-2
    assert np.abs(ld.cpu().numpy() - lp[:, :, 0].cpu().numpy()).max() <= 1e-3


def test_run_to_run_bit_identical_and_workspace_reuse():
    dp = workloads.make_decode(57, 4, 8, 2, 128, 700, (1, 700), "bf16")
    q, kc, vc, sk = decode_inputs(dp)
    ws = torch.empty(fa.decode_workspace_size(q, kc, vc), dtype=torch.uint8, device=DEV)
    outs = [fa.decode(q, kc, vc, sk, scale=dp.scale, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_no_writes_outside_outputs():
    dp = workloads.make_decode(58, 3, 8, 2, 128, 400, (1, 400), "bf16")
    q, kc, vc, sk = decode_inputs(dp)
    pad = 2048
    n = 3 * 8 * 128
    o_buf = torch.full((n + 2 * pad,), 512.0, dtype=torch.bfloat16, device=DEV)
    l_buf = torch.full((24 + 2 * pad,), 777.0, dtype=torch.float32, device=DEV)
    o = o_buf[pad:pad + n].view(3, 8, 128)
    lse = l_buf[pad:pad + 24].view(3, 8)
    fa.decode(q, kc, vc, sk, scale=dp.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o_buf[:pad] == 512.0) and torch.all(o_buf[pad + n:] == 512.0)
    assert torch.all(l_buf[:pad] == 777.0) and torch.all(l_buf[pad + 24:] == 777.0)
    ro, rl = oracle_decode(dp)
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", "decode canaries")


def test_alibi_decode():
    """ALiBi on decode: the query sits at L_b - 1, keys get -m_h (L_b - 1 - j)."""
    dp = workloads.make_decode(58, 6, 16, 4, 128, 3000, (1, 3000), "bf16")
    slopes = [2.0 ** (-8.0 * (h + 1) / 16) for h in range(16)]
    say(f"[decode] ALiBi B=6 Hq=16 Hkv=4 cap=3000")
    o, lse = run_decode(dp, alibi_slopes=slopes)
    ro, rl = oracle_decode(dp, alibi_slopes=slopes)
    check(o, lse, ro, rl, dp.dtype, "ALiBi decode")


def test_alibi_decode_window_and_d64():
    dp = workloads.make_decode(59, 5, 8, 2, 64, 1200, (1, 1200), "bf16", window_left=300)
    slopes = [0.5 * (h + 1) / 8 for h in range(8)]
    o, lse = run_decode(dp, alibi_slopes=slopes)
    ro, rl = oracle_decode(dp, alibi_slopes=slopes)
    check(o, lse, ro, rl, dp.dtype, "ALiBi decode window d64")


def test_long_cache_many_chunks():
    """One sequence of 60000 keys in 128-key chunks: 469 partials, combined in
    many rounds of the combine kernel."""
    dp = workloads.make_decode(161, 2, 8, 2, 128, 60000, (1, 60000), "bf16",
                               lengths=np.array([60000, 33333], dtype=np.int32))
    _case(dp, "long cache, 128-key chunks", chunk_keys=128)
    _case(dp, "long cache, library chunks")


def test_batch_offsets_beyond_2_31_elements():
    """Maximum sizes: caches of 64 sequences x 65536 rows x 8 KV heads x 128
    dims (8 GiB each in bf16), so the last sequence starts 63 x 2^26 elements
    (8 GiB) in.  Sequences 0-62 hold up to 600 seeded rows, the last one is
    full (65536 rows, 64 partial chunks); every other row is NaN."""
    B, cap, Hq, Hkv, d = 64, 65536, 32, 8, 128
    short = workloads.make_decode(191, B - 1, Hq, Hkv, d, 600, (1, 600), "bf16")
    full = workloads.make_decode(192, 1, Hq, Hkv, d, cap, (cap, cap), "bf16")
    say(f"[decode] offsets past 2^31 elements: B={B} cap={cap} last length {int(full.seqlens_k[0])}")
    kc, vc = (torch.full((B, cap, Hkv, d), float("nan"), dtype=torch.bfloat16, device=DEV)
              for _ in range(2))
    kc[:B - 1, :600] = dev_tensor(short.k_cache, "bf16")
    vc[:B - 1, :600] = dev_tensor(short.v_cache, "bf16")
    kc[B - 1] = dev_tensor(full.k_cache[0], "bf16")
    vc[B - 1] = dev_tensor(full.v_cache[0], "bf16")
    assert kc[B - 1].data_ptr() - kc.data_ptr() == (B - 1) * cap * Hkv * d * 2
    q = torch.cat([dev_tensor(short.q, "bf16"), dev_tensor(full.q, "bf16")])
    sk = torch.from_numpy(np.concatenate([short.seqlens_k, full.seqlens_k])).to(DEV)
    o, lse = fa.decode(q, kc, vc, sk, scale=short.scale)
    torch.cuda.synchronize()
    del kc, vc
    torch.cuda.empty_cache()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    ro, rl = oracle_decode(short)
    check(o[:B - 1], lse[:B - 1], ro, rl, "bf16", "short sequences, offsets past 2^31")
    ro, rl = oracle_decode(full)
    check(o[B - 1:], lse[B - 1:], ro, rl, "bf16", "full 65536-row sequence at offset 2^32+")
