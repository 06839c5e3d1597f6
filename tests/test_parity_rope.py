"""GPU parity: RoPE fused into attention (prefill: queries rotated as they
are loaded, keys by the K rotation pass for bf16 or as they are staged for
fp32; decode: the query at L - 1) against the fp64 oracle, which rotates Q
and K, holds them in the input dtype (round to nearest even), and then runs
the plain three-step attention.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import (DEV, check, dev_tensor, oracle_decode, oracle_prefill, prefill_inputs,
                         run_decode, say, to_np)

pytestmark = pytest.mark.gpu


def tables(n_pos, rotary_dim, base=10000.0):
    """cos / sin of position x frequency, frequencies base^(-2p / rotary_dim)."""
    half = rotary_dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / rotary_dim)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _prefill_case(p, rotary_dim, ctx, rows=None, heads=None, alibi=None, base=10000.0):
    Nk = p.k.shape[1]
    cos_t, sin_t = tables(Nk, rotary_dim, base)
    say(f"[rope] {ctx} shape={p.shape} {p.dtype} causal={p.causal} W={p.window_left} "
        f"rotary={rotary_dim}")
    q, k, v, sq, sk = prefill_inputs(p)
    o, lse = fa.prefill(q, k, v, causal=p.causal, window=p.window_left, scale=p.scale,
                        seqlens_q=sq, seqlens_k=sk, rope_cos=torch.from_numpy(cos_t).to(DEV),
                        rope_sin=torch.from_numpy(sin_t).to(DEV),
                        alibi_slopes=None if alibi is None else torch.from_numpy(alibi).to(DEV))
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    ro, rl = oracle.attention(workloads.to_f64(p.q, p.dtype), workloads.to_f64(p.k, p.dtype),
                              workloads.to_f64(p.v, p.dtype), scale=p.scale, causal=p.causal,
                              window_left=p.window_left, seqlens_q=p.seqlens_q,
                              seqlens_k=p.seqlens_k, rows=rows, heads=heads, alibi_slopes=alibi,
                              rope=(cos_t, sin_t, rotary_dim, p.dtype))
    if rows is not None:
        o = o[:, rows][:, :, heads]
        lse = lse[:, heads][:, :, rows]
    check(o, lse, ro, rl, p.dtype, ctx)


@pytest.mark.parametrize("causal", [True, False])
def test_rope_prefill_mha(causal):
    p = workloads.make_prefill(90, 1, 700, 700, 4, 4, 128, "bf16", causal=causal)
    _prefill_case(p, 128, "MHA full rotation")


def test_rope_prefill_gqa_varlen_partial():
    p = workloads.make_prefill(91, 3, 333, 333, 8, 2, 128, "bf16", causal=True,
                               seqlens_k_range=(1, 333), seqlens_q_equal_k=True,
                               poison_padding=True)
    _prefill_case(p, 64, "GQA varlen, rotary 64 of 128")


def test_rope_prefill_fewer_queries_than_keys():
    # queries sit at i + Lk - Lq: the last 100 positions of 900
    p = workloads.make_prefill(92, 2, 100, 900, 4, 1, 128, "bf16", causal=True)
    _prefill_case(p, 128, "Nq 100 < Nk 900, MQA")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_prefill_more_queries_than_keys(causal, dtype):
    """Lq > Lk: rows i < Lq - Lk sit before position 0 and see no key under
    RoPE (O = 0, LSE = -inf); the tables hold exactly Nk rows, so a read at a
    negative position would leave them.  Static extents (Nq 700 > Nk 300, the
    rows before 400 empty) and valid key lengths below the query extent (the
    BERT-shaped call: Nq = Nk = 512, seqlens_k in [128, 512], all query rows
    computed)."""
    d = 128 if dtype == "bf16" else 64
    p = workloads.make_prefill(95, 1, 700, 300, 4, 2, d, dtype, causal=causal)
    _prefill_case(p, d, f"Nq 700 > Nk 300 {dtype}")
    p = workloads.make_prefill(96, 4, 512, 512, 4, 4, 64, dtype, causal=causal,
                               seqlens_k_range=(128, 512), poison_padding=True)
    _prefill_case(p, 64, f"seqlens_k in [128, 512] < Nq 512 {dtype}")


def test_rope_prefill_d64_window_alibi():
    p = workloads.make_prefill(93, 2, 520, 520, 6, 3, 64, "bf16", causal=True, window_left=100)
    _prefill_case(p, 32, "d64 window 100, rotary 32")
    _prefill_case(p, 64, "d64 window 100, rotary 64, ALiBi",
                  alibi=np.linspace(0.01, 0.2, 6).astype(np.float32))


def test_rope_prefill_fp32():
    p = workloads.make_prefill(94, 2, 150, 150, 2, 1, 64, "f32", causal=True,
                               seqlens_k_range=(1, 150), seqlens_q_equal_k=True)
    _prefill_case(p, 32, "fp32 varlen, rotary 32")
    p = workloads.make_prefill(95, 1, 128, 128, 1, 1, 64, "f32")
    _prefill_case(p, 64, "fp32 tiny workload shape, full rotation")


def test_rope_prefill_8k_sampled():
    """The causal N=8192 d=128 workload with RoPE, on sampled rows x heads."""
    p = workloads.make_workload(3)
    rows = np.array([0, 1, 255, 256, 4095, 4096, 8000, 8191])
    _prefill_case(p, 128, "8k causal sampled", rows=rows, heads=np.array([0, 17, 31]),
                  base=500000.0)


def test_rope_identity_tables_change_nothing():
    """cos = 1, sin = 0 leaves every bit of the output unchanged (the
    rotation, the K pass and the copy are exact)."""
    p = workloads.make_prefill(96, 2, 300, 300, 4, 2, 128, "bf16", causal=True,
                               seqlens_k_range=(1, 300), seqlens_q_equal_k=True)
    q, k, v, sq, sk = prefill_inputs(p)
    o1, l1 = fa.prefill(q, k, v, causal=True, scale=p.scale, seqlens_q=sq, seqlens_k=sk)
    ones = torch.ones(300, 64, dtype=torch.float32, device=DEV)
    ws = torch.empty(fa.prefill_workspace_size(q, k, rope_cos=ones, rope_sin=ones),
                     dtype=torch.uint8, device=DEV)
    o2, l2 = fa.prefill(q, k, v, causal=True, scale=p.scale, seqlens_q=sq, seqlens_k=sk,
                        rope_cos=ones, rope_sin=torch.zeros_like(ones), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "paged"])
def test_rope_decode(kind):
    """Decode rotates the query at L - 1; the cache holds keys as stored."""
    say(f"[rope] decode {kind}")
    cos_t, sin_t = tables(1024, 128)      # covers the paged capacity (32 pages of 32)
    c, s = torch.from_numpy(cos_t).to(DEV), torch.from_numpy(sin_t).to(DEV)
    rope = (cos_t, sin_t, 128, "bf16")      # the query is held in bf16 once rotated
    if kind == "bf16":
        dp = workloads.make_decode(97, 6, 8, 2, 128, 1000, (1, 1000), "bf16")
        o, lse = run_decode(dp, rope_cos=c, rope_sin=s)
        ro, rl = oracle.decode(workloads.to_f64(dp.q, "bf16"), workloads.to_f64(dp.k_cache, "bf16"),
                               workloads.to_f64(dp.v_cache, "bf16"), dp.seqlens_k, scale=dp.scale,
                               rope_q=rope)
    elif kind == "fp8":
        from gpu_helpers import run_decode_fp8
        dp = workloads.make_decode(98, 6, 8, 2, 128, 1000, (1, 1000), "bf16", kv_dtype="fp8_e4m3")
        o, lse = run_decode_fp8(dp, rope_cos=c, rope_sin=s)
        ro, rl = oracle.decode(workloads.to_f64(dp.q, "bf16"),
                               oracle.dequantize_kv(dp.k_cache, dp.k_scale),
                               oracle.dequantize_kv(dp.v_cache, dp.v_scale), dp.seqlens_k,
                               scale=dp.scale, rope_q=rope)
    else:
        from gpu_helpers import run_decode_paged
        pp = workloads.make_decode_paged(99, 6, 8, 2, 128, 1000, (1, 1000), 32, "bf16",
                                         window_left=200)
        o, lse = run_decode_paged(pp, rope_cos=c, rope_sin=s)
        L = pp.seqlens_k
        ro = np.zeros((6, 8, 128))
        rl = np.zeros((6, 8))
        q = workloads.to_f64(pp.q, "bf16")
        for b in range(6):
            kb = oracle.gather_paged(workloads.to_f64(pp.k_pool, "bf16"), pp.block_table[b], int(L[b]))
            vb = oracle.gather_paged(workloads.to_f64(pp.v_pool, "bf16"), pp.block_table[b], int(L[b]))
            ob, lb = oracle.decode(q[b:b + 1], kb[None], vb[None], [int(L[b])], scale=pp.scale,
                                   window_left=200, rope_q=rope)
            ro[b], rl[b] = ob[0], lb[0]
    check(o, lse, ro, rl, "bf16", f"decode RoPE {kind}")


def test_rope_k_pass_writes_only_its_workspace():
    """The K rotation pass writes the valid rows of its workspace and nothing
    around it; the workspace rows past a sequence's key length stay as they
    were (the attention kernel never reads them)."""
    p = workloads.make_prefill(130, 2, 200, 200, 4, 2, 128, "bf16", causal=True,
                               seqlens_k_range=(50, 200), seqlens_q_equal_k=True)
    cos_t, sin_t = tables(200, 128)
    c, s = torch.from_numpy(cos_t).to(DEV), torch.from_numpy(sin_t).to(DEV)
    q, k, v, sq, sk = prefill_inputs(p)
    need = fa.prefill_workspace_size(q, k, rope_cos=c, rope_sin=s)
    assert need == 2 * 200 * 2 * 128 * 2
    pad = 4096
    buf = torch.full((need + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = buf[pad:pad + need]
    say("[rope] K pass canaries")
    o, lse = fa.prefill(q, k, v, causal=True, scale=p.scale, seqlens_q=sq, seqlens_k=sk,
                        rope_cos=c, rope_sin=s, workspace=ws)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 0xA5) and np.all(host[pad + need:] == 0xA5)
    rows = host[pad:pad + need].view(np.uint16).reshape(2, 200, 2, 128)
    for b in range(2):
        L = int(p.seqlens_k[b])
        assert np.all(rows[b, L:] == 0xA5A5)          # untouched past the valid length
        want = oracle.rope_rotate(workloads.to_f64(p.k[b, :L].reshape(L * 2, 128), "bf16"),
                                  np.repeat(np.arange(L), 2), cos_t, sin_t, 128, "bf16")
        got = workloads.bf16_bits_to_f32(rows[b, :L].reshape(L * 2, 128)).astype(np.float64)
        # the kernel rounds x c - y s computed in fp32, the oracle the exact value: at
        # most one bf16 step apart, and equal almost everywhere
        step = np.abs(want) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(got - want) <= step)
        assert np.mean(got == want) > 0.99
    ro, rl = oracle.attention(workloads.to_f64(p.q, "bf16"), workloads.to_f64(p.k, "bf16"),
                              workloads.to_f64(p.v, "bf16"), scale=p.scale, causal=True,
                              seqlens_q=p.seqlens_q, seqlens_k=p.seqlens_k,
                              rope=(cos_t, sin_t, 128, "bf16"))
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", "RoPE canaries")


@pytest.mark.parametrize("Hq,Hkv,d,rdim", [(8, 4, 128, 64), (4, 2, 64, 32), (8, 2, 64, 64)])
def test_rope_decode_fp8_partial_rotary(Hq, Hkv, d, rdim):
    """FP8 cache with RoPE over the first rdim dims only, for head dims 128
    and 64 and GQA groups of 2 and 4: the query's rotated and unrotated dims
    sit in the matrix-core operand layout of the FP8 path."""
    from gpu_helpers import run_decode_fp8
    say(f"[rope] decode fp8 Hq{Hq} Hkv{Hkv} d{d} rotary {rdim}")
    cos_t, sin_t = tables(1000, rdim)
    c, s = torch.from_numpy(cos_t).to(DEV), torch.from_numpy(sin_t).to(DEV)
    dp = workloads.make_decode(140 + Hq + d + rdim, 5, Hq, Hkv, d, 1000, (1, 1000), "bf16",
                               kv_dtype="fp8_e4m3")
    o, lse = run_decode_fp8(dp, rope_cos=c, rope_sin=s)
    ro, rl = oracle.decode(workloads.to_f64(dp.q, "bf16"), oracle.dequantize_kv(dp.k_cache, dp.k_scale),
                           oracle.dequantize_kv(dp.v_cache, dp.v_scale), dp.seqlens_k, scale=dp.scale,
                           rope_q=(cos_t, sin_t, rdim, "bf16"))
    check(o, lse, ro, rl, "bf16", f"decode RoPE fp8 d{d} rotary {rdim}")
