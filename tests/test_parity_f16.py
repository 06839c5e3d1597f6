"""GPU parity for IEEE half (FA_DTYPE_F16) inputs: the prefill (half MFMA,
fp32 accumulation, P rounded to half), the K rotation pass, the decode (half
dot products) over plain, paged and FP8 caches, against the fp64 oracle on
the same half values.  Tolerances are the 16-bit ones of the bf16 tests.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import (DEV, check, oracle_decode, oracle_decode_fp8, oracle_decode_paged,
                         oracle_prefill, run_decode, run_decode_fp8, run_decode_paged, run_prefill,
                         say, to_np, prefill_inputs)

pytestmark = pytest.mark.gpu


def _case(p, ctx, **kw):
    say(f"[f16] {ctx} shape={p.shape} causal={p.causal} W={p.window_left}")
    o, lse = run_prefill(p, **kw)
    ro, rl = oracle_prefill(p, alibi_slopes=kw.get("alibi_slopes"))
    check(o, lse, ro, rl, "f16", ctx)


@pytest.mark.parametrize("causal", [True, False])
def test_f16_mha(causal):
    _case(workloads.make_prefill(170, 1, 700, 700, 4, 4, 128, "f16", causal=causal), "MHA")


def test_f16_gqa_varlen_window_d64():
    _case(workloads.make_prefill(171, 3, 333, 333, 8, 2, 128, "f16", causal=True, window_left=100,
                                 seqlens_k_range=(1, 333), seqlens_q_equal_k=True,
                                 poison_padding=True), "GQA varlen window")
    _case(workloads.make_prefill(172, 2, 300, 257, 6, 3, 64, "f16", causal=True), "d64 Nk < Nq")


def test_f16_bert_workload_shape():
    w = dict(workloads.WORKLOADS[2])
    p = workloads.make_prefill(w["seed"], w["B"], w["Nq"], w["Nk"], w["Hq"], w["Hkv"], w["d"],
                               "f16", seqlens_k_range=w["seqlens_k_range"])
    _case(p, "BERT-base B8 H12 N512 d64, key lengths U[128, 512], half")


def test_f16_large_scores_stay_finite():
    """Scores far above the first tile's: P must not overflow half (the fast
    path's bound is lower for half)."""
    p = workloads.make_prefill(173, 1, 300, 300, 2, 2, 128, "f16", causal=True)
    k = workloads.to_f64(p.k, "f16") + 4.0
    q = workloads.to_f64(p.q, "f16") + 2.0
    p.k = workloads._store(k.astype(np.float32), "f16")
    p.q = workloads._store(q.astype(np.float32), "f16")
    _case(p, "large score offsets")


def test_f16_alibi_mask_rope():
    p = workloads.make_prefill(174, 2, 260, 260, 4, 2, 128, "f16", causal=True)
    _case(p, "ALiBi", alibi_slopes=[0.5, 0.1, 0.02, 0.004])
    half = 64
    inv = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.arange(260, dtype=np.float64)[:, None] * inv[None, :]
    cos_t, sin_t = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    say("[f16] RoPE")
    q, k, v, sq, sk = prefill_inputs(p)
    o, lse = fa.prefill(q, k, v, causal=True, scale=p.scale, rope_cos=torch.from_numpy(cos_t).to(DEV),
                        rope_sin=torch.from_numpy(sin_t).to(DEV))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(workloads.to_f64(p.q, "f16"), workloads.to_f64(p.k, "f16"),
                              workloads.to_f64(p.v, "f16"), scale=p.scale, causal=True,
                              rope=(cos_t, sin_t, 128, "f16"))
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "f16", "RoPE")
    say("[f16] explicit mask")
    m = np.random.default_rng(175).standard_normal((2, 1, 260, 260)).astype(np.float32)
    mt = torch.from_numpy(m).to(torch.float16).to(DEV)
    o, lse = fa.prefill(q, k, v, causal=True, scale=p.scale, attn_mask=mt)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(workloads.to_f64(p.q, "f16"), workloads.to_f64(p.k, "f16"),
                              workloads.to_f64(p.v, "f16"), scale=p.scale, causal=True,
                              attn_mask=mt.float().cpu().numpy().astype(np.float64))
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "f16", "mask")


def test_f16_decode_plain_paged_fp8():
    dp = workloads.make_decode(176, 6, 8, 2, 128, 1000, (1, 1000), "f16", window_left=300)
    say("[f16] decode plain")
    o, lse = run_decode(dp)
    ro, rl = oracle_decode(dp)
    check(o, lse, ro, rl, "f16", "decode")
    pp = workloads.make_decode_paged(177, 6, 8, 2, 128, 1000, (1, 1000), 32, "f16")
    say("[f16] decode paged")
    o, lse = run_decode_paged(pp)
    ro, rl = oracle_decode_paged(pp)
    check(o, lse, ro, rl, "f16", "decode paged")
    fp = workloads.make_decode(178, 6, 8, 2, 64, 1000, (1, 1000), "f16", kv_dtype="fp8_e4m3")
    say("[f16] decode FP8 cache")
    o, lse = run_decode_fp8(fp)
    ro, rl = oracle_decode_fp8(fp)
    check(o, lse, ro, rl, "f16", "decode FP8 cache, half q")


def test_every_e4m3_code_into_half():
    """All 256 codes through the value path with a half query: exact values
    come back (half holds every E4M3 value)."""
    from gpu_helpers import fp8_tensor
    say("[f16] all 256 E4M3 codes into half")
    codes = np.arange(256, dtype=np.uint8).reshape(2, 1, 1, 128)
    q = torch.zeros((2, 1, 128), dtype=torch.float16, device=DEV)
    kc = fp8_tensor(np.full((2, 1, 1, 128), 0x38, dtype=np.uint8))
    o, lse = fa.decode(q, kc, fp8_tensor(codes), torch.ones(2, dtype=torch.int32, device=DEV),
                       k_scale=[1.0], v_scale=[1.0])
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64).reshape(256)
    want = oracle.fp8_e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
