"""GPU checks against closed forms: each expected value follows from the
definition of attention alone (only the visibility predicate is taken from
the oracle, which is itself pinned against hand-written tables).

* Q = 0: every visible key has the same score, so O_i is the mean of the
  visible V rows and LSE_i = ln |visible(i)|.
* identical V rows: O_i = v for every row that sees a key; a column of ones
  in V gives a column of ones in O (up to the bf16 rounding of P, which the
  matrix product uses while the row sum keeps fp32).
* a single visible key (causal row 0): O_0 = V_0 bit for bit and
  LSE_0 = scale q_0 . k_0.
* a joint permutation of the K and V rows leaves a non-causal result
  unchanged.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import DEV, dev_tensor, say, to_np

pytestmark = pytest.mark.gpu


def _zero_q(p):
    p.q = np.zeros_like(p.q)
    return p


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kw", [dict(causal=True), dict(causal=True, window_left=50),
                                dict(window_left=30), dict()])
def test_zero_query_gives_mean_and_log_count(dtype, kw):
    p = _zero_q(workloads.make_prefill(150, 2, 190, 230, 4, 2, 128 if dtype == "bf16" else 64,
                                       dtype, seqlens_k_range=(1, 230), **kw))
    say(f"[closed] Q = 0 {dtype} {kw}")
    q, k, v = (dev_tensor(x, dtype) for x in (p.q, p.k, p.v))
    sk = torch.from_numpy(p.seqlens_k).to(DEV)
    o, lse = fa.prefill(q, k, v, scale=p.scale, seqlens_k=sk, **{("window" if a == "window_left"
                                                                   else a): b for a, b in kw.items()})
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    vf = workloads.to_f64(p.v, dtype)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for b in range(2):
        Lk = int(p.seqlens_k[b])
        vis = oracle.visible_matrix(np.arange(190), 230, 190, Lk, kw.get("causal", False),
                                    kw.get("window_left", -1))
        for h in range(4):
            for i in range(190):
                n = int(vis[i].sum())
                if n == 0:
                    assert np.all(o[b, i, h] == 0) and lse[b, h, i] == -np.inf
                    continue
                mean = vf[b, vis[i], h // 2].mean(axis=0)
                assert np.abs(o[b, i, h] - mean).max() <= tol
                assert abs(lse[b, h, i] - math.log(n)) <= 1e-5


def test_zero_query_decode():
    dp = workloads.make_decode(151, 5, 8, 2, 128, 700, (1, 700), "bf16", window_left=90)
    dp.q = np.zeros_like(dp.q)
    say("[closed] decode Q = 0, window 90")
    q, kc, vc = (dev_tensor(x, "bf16") for x in (dp.q, dp.k_cache, dp.v_cache))
    o, lse = fa.decode(q, kc, vc, torch.from_numpy(dp.seqlens_k).to(DEV), window=90)
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    vf = workloads.to_f64(dp.v_cache, "bf16")
    for b in range(5):
        L = int(dp.seqlens_k[b])
        lo = max(0, L - 90)
        for h in range(8):
            assert np.abs(o[b, h] - vf[b, lo:L, h // 4].mean(axis=0)).max() <= 2e-2
            assert abs(lse[b, h] - math.log(L - lo)) <= 1e-5


def test_identical_v_rows_and_ones_column():
    p = workloads.make_prefill(152, 2, 300, 300, 4, 2, 128, "bf16", causal=True)
    v = workloads.bf16_bits_to_f32(p.v)
    v[:, :, :, :] = v[:, :1, :, :]                 # every row equals row 0 (per KV head)
    v[:, :, :, 5] = 1.0                            # and dim 5 is all ones
    p.v = workloads.f32_to_bf16_bits(v)
    say("[closed] identical V rows, ones column")
    q, k, vv = (dev_tensor(x, "bf16") for x in (p.q, p.k, p.v))
    o, _ = fa.prefill(q, k, vv, causal=True, scale=p.scale)
    torch.cuda.synchronize()
    o = to_np(o)
    want = workloads.bf16_bits_to_f32(p.v)[:, 0].astype(np.float64)   # [B, Hkv, d]
    for h in range(4):
        np.testing.assert_allclose(o[:, :, h], np.broadcast_to(want[:, None, h // 2], o[:, :, h].shape),
                                   rtol=2 ** -7, atol=1e-3)
    assert np.abs(o[..., 5] - 1.0).max() <= 2 ** -7


def test_single_visible_key_is_exact():
    p = workloads.make_prefill(153, 2, 100, 100, 4, 4, 128, "bf16", causal=True)
    say("[closed] causal row 0 = V_0")
    q, k, v = (dev_tensor(x, "bf16") for x in (p.q, p.k, p.v))
    o, lse = fa.prefill(q, k, v, causal=True, scale=p.scale)
    torch.cuda.synchronize()
    assert torch.equal(o[:, 0].view(torch.int16), v[:, 0].view(torch.int16))
    qf = workloads.to_f64(p.q, "bf16")[:, 0]
    kf = workloads.to_f64(p.k, "bf16")[:, 0]
    want = float(np.float32(p.scale)) * np.einsum("bhd,bhd->bh", qf, kf)
    assert np.abs(lse[:, :, 0].cpu().numpy() - want).max() <= 1e-4


def test_joint_permutation_of_keys_and_values():
    p = workloads.make_prefill(154, 1, 200, 333, 4, 2, 128, "bf16")
    perm = np.random.default_rng(155).permutation(333)
    say("[closed] joint permutation of K and V rows")
    q, k, v = (dev_tensor(x, "bf16") for x in (p.q, p.k, p.v))
    kp, vp = (dev_tensor(np.ascontiguousarray(x[:, perm]), "bf16") for x in (p.k, p.v))
    o1, l1 = fa.prefill(q, k, v, scale=p.scale)
    o2, l2 = fa.prefill(q, kp, vp, scale=p.scale)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-4
