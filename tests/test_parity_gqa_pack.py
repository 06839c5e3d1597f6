"""GPU parity of the packed GQA prefill: with bf16 and head_dim 128, the
query heads of a KV group share a workgroup (up to 8 of them, 256 / 8 = 32
positions each).  Against the fp64 oracle on every output, for groups of 2,
4, 8 and 16 heads under causal, window, valid-length and cross-length
problems and with every bias at once; and bit for bit against the same
problem run as plain multi-head attention (K and V copied once per query
head), which takes the one-head-per-workgroup kernel: each wavefront visits
the same key tiles in the same order either way.  With more work items
than CUs the packed kernel runs in its persistent form (one workgroup per
CU walking the items); that form is checked the same two ways.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import DEV, check, oracle_prefill, prefill_inputs, run_prefill, say, to_np

pytestmark = pytest.mark.gpu


def _case(p, ctx, **kw):
    say(f"[gqa pack] {ctx} shape(B,Nq,Nk,Hq,Hkv,d)={p.shape} causal={p.causal} W={p.window_left} "
        f"seqlens_q={p.seqlens_q is not None} seqlens_k={p.seqlens_k is not None}")
    o, lse = run_prefill(p, **kw)
    ro, rl = oracle_prefill(p, alibi_slopes=kw.get("alibi_slopes"))
    check(o, lse, ro, rl, p.dtype, ctx)
    return o, lse


@pytest.mark.parametrize("group", [2, 4, 8, 16])
@pytest.mark.parametrize("kind", ["causal", "window", "varlen", "noncausal_cross"])
def test_packed_groups(group, kind):
    Hkv = 2
    Hq = Hkv * group
    if kind == "causal":
        p = workloads.make_prefill(300 + group, 2, 300, 300, Hq, Hkv, 128, "bf16", causal=True)
    elif kind == "window":
        p = workloads.make_prefill(310 + group, 2, 333, 333, Hq, Hkv, 128, "bf16", causal=True,
                                   window_left=70)
    elif kind == "varlen":
        p = workloads.make_prefill(320 + group, 3, 290, 290, Hq, Hkv, 128, "bf16", causal=True,
                                   seqlens_k_range=(1, 290), seqlens_q_equal_k=True,
                                   poison_padding=True)
    else:
        p = workloads.make_prefill(330 + group, 2, 150, 260, Hq, Hkv, 128, "bf16")
    _case(p, f"group {group} {kind}")


def test_packed_with_every_bias():
    """ALiBi, RoPE and an explicit mask together with a window and Lq < Lk,
    group 4 (packed 4 heads x 64 positions)."""
    p = workloads.make_prefill(340, 2, 200, 330, 8, 2, 128, "bf16", causal=True, window_left=150)
    slopes = np.linspace(0.02, 0.3, 8).astype(np.float32)
    rng = np.random.default_rng(341)
    mask = rng.standard_normal((2, 8, 200, 330))
    mask[:, :, :, 300:] = -np.inf
    mbits = workloads.f32_to_bf16_bits(mask.astype(np.float32))
    mt = torch.from_numpy(mbits.view(np.int16)).view(torch.bfloat16).to(DEV)
    mv = workloads.bf16_bits_to_f32(mbits).astype(np.float64)
    half = 64
    inv = 10000.0 ** (-np.arange(half, dtype=np.float64) * 2.0 / 128)
    ang = np.arange(330, dtype=np.float64)[:, None] * inv[None, :]
    cos_t, sin_t = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    c, s = torch.from_numpy(cos_t).to(DEV), torch.from_numpy(sin_t).to(DEV)
    q, k, v, sq, sk = prefill_inputs(p)
    ws = torch.empty(fa.prefill_workspace_size(q, k, rope_cos=c, rope_sin=s), dtype=torch.uint8,
                     device=DEV)
    say("[gqa pack] group 4 with ALiBi, RoPE, mask, window 150, Nq 200 < Nk 330")
    o, lse = fa.prefill(q, k, v, causal=True, window=150, scale=p.scale,
                        alibi_slopes=torch.from_numpy(slopes).to(DEV), rope_cos=c, rope_sin=s,
                        workspace=ws, attn_mask=mt)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(workloads.to_f64(p.q, "bf16"), workloads.to_f64(p.k, "bf16"),
                              workloads.to_f64(p.v, "bf16"), scale=p.scale, causal=True,
                              window_left=150, alibi_slopes=slopes, attn_mask=mv,
                              rope=(cos_t, sin_t, 128, "bf16"))
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", "packed, every bias")


@pytest.mark.parametrize("group,kw", [(4, dict(causal=True, window_left=100)),
                                      (8, dict(causal=True)),
                                      (2, dict(seqlens_k_range=(50, 400)))])
def test_packed_bit_identical_to_per_head_kernel(group, kw):
    """The packed kernel against plain MHA on K and V copied per query head."""
    Hkv = 2
    p = workloads.make_prefill(350 + group, 2, 400, 400, Hkv * group, Hkv, 128, "bf16", **kw)
    say(f"[gqa pack] bit identity, group {group} {kw}")
    o1, l1 = run_prefill(p)
    mha = workloads.PrefillProblem("bf16", p.q, np.repeat(p.k, group, axis=2),
                                   np.repeat(p.v, group, axis=2), p.scale, p.causal,
                                   p.window_left, p.seqlens_q, p.seqlens_k)
    o2, l2 = run_prefill(mha)
    assert np.array_equal(o1, o2), "packed GQA output differs from the per-head kernel"
    assert np.array_equal(l1, l2), "packed GQA LSE differs from the per-head kernel"


def _persistent_problem(seed, **kw):
    # B2 Hq32 Hkv8 N1100, group 4: 4 heads x 64 positions per workgroup, so
    # 18 position blocks x 8 KV heads x 2 sequences = 288 work items, more than
    # the CUs of the device: the persistent form runs (one workgroup per CU,
    # a second, partial round in snake order)
    return workloads.make_prefill(seed, 2, 1100, 1100, 32, 8, 128, "bf16", **kw)


@pytest.mark.parametrize("kind", ["causal", "window", "varlen_with_empty"])
def test_persistent_packed_form(kind):
    """The persistent form of the packed kernel (more work items than CUs)
    against the oracle on every output, including an empty sequence whose
    query rows the next-item Q staging clamps."""
    assert torch.cuda.get_device_properties(0).multi_processor_count < 288
    if kind == "causal":
        p = _persistent_problem(360, causal=True)
    elif kind == "window":
        p = _persistent_problem(361, causal=True, window_left=300)
    else:
        p = _persistent_problem(362, causal=True, seqlens_k_range=(1, 1100), seqlens_q_equal_k=True,
                                poison_padding=True)
        nan = workloads.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
        p.seqlens_k[0] = 0
        p.seqlens_q[0] = 0
        p.q[0] = nan
        p.k[0] = nan
        p.v[0] = nan
    _case(p, f"persistent {kind}")


def test_persistent_form_bit_identical_to_per_head_kernel():
    """The persistent packed kernel against plain MHA (K and V copied per
    query head, one head per workgroup, one workgroup per item)."""
    p = _persistent_problem(363, causal=True, window_left=500)
    say("[gqa pack] persistent form, bit identity against the per-head kernel")
    o1, l1 = run_prefill(p)
    mha = workloads.PrefillProblem("bf16", p.q, np.repeat(p.k, 4, axis=2), np.repeat(p.v, 4, axis=2),
                                   p.scale, p.causal, p.window_left, p.seqlens_q, p.seqlens_k)
    o2, l2 = run_prefill(mha)
    assert np.array_equal(o1, o2), "persistent packed output differs from the per-head kernel"
    assert np.array_equal(l1, l2), "persistent packed LSE differs from the per-head kernel"
