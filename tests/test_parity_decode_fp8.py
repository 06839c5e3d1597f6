"""GPU parity: fa_decode_fwd over an FP8 E4M3 KV cache (per-KV-head scales),
contiguous and paged, against the fp64 oracle on the dequantized cache.
Rows past each sequence's length hold the E4M3 NaN code, so a read the
lengths do not allow poisons the output.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import (DEV, check, dev_tensor, fp8_tensor, oracle_decode_fp8,
                         oracle_decode_paged_fp8, run_decode_fp8, run_decode_paged_fp8, say,
                         to_np)

pytestmark = pytest.mark.gpu


def _case(dp, ctx, alibi_slopes=None, **kw):
    say(f"[fp8] {ctx} B={dp.q.shape[0]} Hq={dp.q.shape[1]} Hkv={dp.k_cache.shape[2]} "
        f"d={dp.q.shape[2]} cap={dp.k_cache.shape[1]} W={dp.window_left} {kw}")
    o, lse = run_decode_fp8(dp, alibi_slopes=alibi_slopes, **kw)
    ro, rl = oracle_decode_fp8(dp, alibi_slopes=alibi_slopes)
    check(o, lse, ro, rl, "bf16", ctx)


@pytest.mark.parametrize("v_scale", [1.0, 0.5])
def test_every_e4m3_code_through_the_value_path(v_scale):
    """One key per sequence, so O is that key's V row times v_scale: all 256
    codes come back as their exact values (bf16 holds every E4M3 value), NaN
    codes as NaN -- a check of the hardware conversion against the E4M3
    definition."""
    say(f"[fp8] all 256 codes, v_scale={v_scale}")
    codes = np.arange(256, dtype=np.uint8).reshape(2, 1, 1, 128)
    q = dev_tensor(workloads.f32_to_bf16_bits(np.zeros((2, 1, 128), np.float32)), "bf16")
    kc = fp8_tensor(np.full((2, 1, 1, 128), 0x38, dtype=np.uint8))
    vc = fp8_tensor(codes)
    sk = torch.ones(2, dtype=torch.int32, device=DEV)
    o, lse = fa.decode(q, kc, vc, sk, k_scale=[1.0], v_scale=[v_scale])
    torch.cuda.synchronize()
    got = to_np(o).reshape(256)
    want = v_scale * oracle.fp8_e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin]), np.nonzero(got[fin] != want[fin])
    assert np.all(lse.cpu().numpy() == 0.0)          # one key with score 0: LSE = ln 1


def test_fp8_decode_workload_shape():
    """The decode workload (B64 Hq32 Hkv8 d128, L ~ U[512, 8192]) with an FP8 cache."""
    w = workloads.WORKLOADS[5]
    dp = workloads.make_decode(w["seed"], w["B"], w["Hq"], w["Hkv"], w["d"], w["capacity"],
                               w["len_range"], "bf16", kv_dtype="fp8_e4m3")
    _case(dp, "decode workload, FP8 cache")


@pytest.mark.parametrize("chunk", [0, 128, 512])
def test_fp8_lengths_around_edges(chunk):
    lengths = np.array([1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 511, 512, 513, 0, 1000],
                       dtype=np.int32)
    dp = workloads.make_decode(70, len(lengths), 8, 2, 128, 1000, (1, 1000), "bf16",
                               lengths=lengths, kv_dtype="fp8_e4m3")
    _case(dp, f"FP8 lengths at edges, chunk={chunk}", chunk_keys=chunk)


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 8, 128), (32, 4, 128), (8, 1, 128), (12, 4, 64),
                                      (6, 2, 64), (8, 4, 128), (4, 2, 64), (16, 2, 128)])
def test_fp8_gqa_and_head_dim(Hq, Hkv, d):
    dp = workloads.make_decode(71 + Hq, 5, Hq, Hkv, d, 900, (1, 900), "bf16",
                               kv_dtype="fp8_e4m3")
    _case(dp, f"FP8 Hq{Hq} Hkv{Hkv} d{d}")


@pytest.mark.parametrize("W", [1, 100, 5000])
def test_fp8_window_and_alibi(W):
    dp = workloads.make_decode(72, 6, 8, 2, 128, 1200, (1, 1200), "bf16", window_left=W,
                               kv_dtype="fp8_e4m3")
    _case(dp, f"FP8 window {W}")
    _case(dp, f"FP8 window {W} ALiBi", alibi_slopes=np.linspace(0.02, 0.2, 8).astype(np.float32))


@pytest.mark.parametrize("page", [16, 48, 64, 256])
def test_fp8_paged(page):
    # 16- and 48-row pages take 16-key tiles, 64 and 256 take 32-key tiles
    pp = workloads.make_decode_paged(73, 9, 8, 2, 128, 1100, (1, 1100), page, "bf16",
                                     window_left=70 if page in (48, 64) else -1,
                                     kv_dtype="fp8_e4m3")
    say(f"[fp8] paged page={page} W={pp.window_left}")
    o, lse = run_decode_paged_fp8(pp)
    ro, rl = oracle_decode_paged_fp8(pp)
    check(o, lse, ro, rl, "bf16", f"FP8 paged, page {page}")


def test_fp8_paged_bit_identical_to_contiguous():
    lengths = np.array([1, 17, 300, 1024, 0, 999], dtype=np.int32)
    dp = workloads.make_decode(74, 6, 8, 2, 128, 1024, (1, 1024), "bf16", lengths=lengths,
                               kv_dtype="fp8_e4m3")
    pp = workloads.make_decode_paged(74, 6, 8, 2, 128, 1024, (1, 1024), 32, "bf16",
                                     lengths=lengths, kv_dtype="fp8_e4m3")
    say("[fp8] paged vs contiguous, bitwise")
    o1, l1 = run_decode_fp8(dp)
    o2, l2 = run_decode_paged_fp8(pp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fp8_scales_and_growing_scores():
    """Per-head scales far from 1 (tiny K scale, large V scale), and keys whose
    scores climb fast enough to move every wavefront's reference."""
    dp = workloads.make_decode(75, 4, 8, 2, 128, 1500, (600, 1500), "bf16", kv_dtype="fp8_e4m3")
    dp.k_scale = (dp.k_scale * np.array([1e-3, 40.0], np.float32)).astype(np.float32)
    dp.v_scale = (dp.v_scale * np.array([20.0, 1e-2], np.float32)).astype(np.float32)
    _case(dp, "FP8 extreme scales")
    # head 1 (k_scale x40) climbs: ramp the first dims of K with position
    q = workloads.bf16_bits_to_f32(dp.q)
    q[:, 4:8, :] = np.abs(q[:, 4:8, :]) + 0.5
    dp.q = workloads.f32_to_bf16_bits(q)
    k = oracle.fp8_e4m3_value(dp.k_cache)
    ramp = np.clip(np.arange(1500, dtype=np.float64)[None, :, None, None] / 1500.0 * 400.0, 0, 448)
    k[:, :, 1:2, :16] = np.where(np.isnan(k[:, :, 1:2, :16]), np.nan, ramp)
    dp.k_cache = np.where(np.isnan(k), workloads.FP8_E4M3_QNAN,
                          workloads.f32_to_fp8_e4m3_codes(np.nan_to_num(k).astype(np.float32)))
    _case(dp, "FP8 growing scores")


@pytest.mark.parametrize("d", [128, 64])
def test_every_e4m3_code_over_two_kv_heads(d):
    """Two KV heads with their own V scales: their V rows hold all 256 codes
    between them, one key per sequence, so each query head's O is its KV
    head's V row times that head's scale: every code comes back as its exact
    value, NaN codes as NaN (through the matrix-core P.V of 32-key tiles)."""
    say(f"[fp8] all 256 codes over two KV heads, d={d}")
    B = 256 // (2 * d)
    codes = np.arange(256, dtype=np.uint8).reshape(B, 1, 2, d)
    q = dev_tensor(workloads.f32_to_bf16_bits(np.zeros((B, 2, d), np.float32)), "bf16")
    kc = fp8_tensor(np.full((B, 1, 2, d), 0x38, dtype=np.uint8))
    vc = fp8_tensor(codes)
    sk = torch.ones(B, dtype=torch.int32, device=DEV)
    o, lse = fa.decode(q, kc, vc, sk, k_scale=[1.0, 1.0], v_scale=[1.0, 0.5])
    torch.cuda.synchronize()
    got = to_np(o).reshape(B, 2, d)
    want = oracle.fp8_e4m3_value(codes.reshape(B, 2, d)) * np.array([1.0, 0.5])[None, :, None]
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin]), np.nonzero(got[fin] != want[fin])


@pytest.mark.parametrize("Hq,Hkv,d", [(16, 4, 128), (8, 2, 64), (4, 4, 128)])
def test_fp8_cache_with_a_head_stride(Hq, Hkv, d):
    """The same cache read two ways: as stored and through a view whose head
    stride is 2 d (every other slot of a wider buffer, NaN codes between).
    Both match the oracle."""
    dp = workloads.make_decode(76 + Hq + d, 7, Hq, Hkv, d, 1300, (1, 1300), "bf16",
                               kv_dtype="fp8_e4m3")
    _case(dp, f"FP8 Hq{Hq} Hkv{Hkv} d{d}")
    B, cap = dp.k_cache.shape[:2]
    views = []
    for c in (dp.k_cache, dp.v_cache):
        wide = np.full((B, cap, Hkv, 2 * d), workloads.FP8_E4M3_QNAN, dtype=np.uint8)
        wide[..., :d] = c
        views.append(fp8_tensor(wide)[..., :d])
    assert views[0].stride(2) == 2 * d
    q = dev_tensor(dp.q, dp.dtype)
    sk = torch.from_numpy(dp.seqlens_k).to(DEV)
    say(f"[fp8] through a view with head stride 2 d, Hq{Hq} Hkv{Hkv} d{d}")
    o, lse = fa.decode(q, views[0], views[1], sk, scale=dp.scale,
                       k_scale=torch.from_numpy(dp.k_scale).to(DEV),
                       v_scale=torch.from_numpy(dp.v_scale).to(DEV))
    torch.cuda.synchronize()
    ro, rl = oracle_decode_fp8(dp)
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", "FP8 head-strided view")
