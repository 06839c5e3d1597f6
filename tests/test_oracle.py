"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: hand-written
visibility tables, closed forms, a scalar brute-force loop, library
routines (torch SDPA, scipy logsumexp) and invariants the mathematics fixes.
A plausible slip in the oracle (a dropped mask term, a wrong sign of the
causal offset, a transposed operand, a missing max subtraction, a wrong GQA
map, a log base) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(p):
    return (workloads.to_f64(p.q, p.dtype), workloads.to_f64(p.k, p.dtype),
            workloads.to_f64(p.v, p.dtype))


# ---------------------------------------------------------------------------
# P11: brute force on 4x4 with literal visibility tables
# ---------------------------------------------------------------------------
# (causal, window_left, seqlen_q, seqlen_k) -> visible[i][j], written by hand
LITERAL_4x4 = {
    (False, -1, 4, 4): [[1, 1, 1, 1]] * 4,
    (True, -1, 4, 4): [[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 1, 1, 1]],
    (True, 1, 4, 4): [[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1]],
    (True, 2, 4, 4): [[1, 0, 0, 0], [1, 1, 0, 0], [0, 1, 1, 0], [0, 0, 1, 1]],
    (True, 3, 4, 4): [[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [0, 1, 1, 1]],
    (True, 4, 4, 4): [[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 1, 1, 1]],
    (False, 2, 4, 4): [[1, 1, 1, 1], [1, 1, 1, 1], [0, 1, 1, 1], [0, 0, 1, 1]],
    (False, -1, 4, 2): [[1, 1, 0, 0]] * 4,
    (False, -1, 4, 0): [[0, 0, 0, 0]] * 4,
    (False, -1, 2, 4): [[1, 1, 1, 1], [1, 1, 1, 1], [0, 0, 0, 0], [0, 0, 0, 0]],
    (False, -1, 0, 4): [[0, 0, 0, 0]] * 4,
    # bottom-right causal, fewer keys than queries: rows 0 and 1 see nothing
    (True, -1, 4, 2): [[0, 0, 0, 0], [0, 0, 0, 0], [1, 0, 0, 0], [1, 1, 0, 0]],
    # bottom-right causal, fewer queries than keys
    (True, -1, 2, 4): [[1, 1, 1, 0], [1, 1, 1, 1], [0, 0, 0, 0], [0, 0, 0, 0]],
    (True, -1, 2, 2): [[1, 0, 0, 0], [1, 1, 0, 0], [0, 0, 0, 0], [0, 0, 0, 0]],
    (True, 2, 3, 4): [[1, 1, 0, 0], [0, 1, 1, 0], [0, 0, 1, 1], [0, 0, 0, 0]],
    (True, 1, 4, 3): [[0, 0, 0, 0], [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0]],
}


def _scalar_attention(q, k, v, scale, vis):
    """Scalar loop: softmax weights with math.exp, no NumPy reductions."""
    n_q, d = len(q), len(q[0])
    out, lse = [], []
    for i in range(n_q):
        scores = []
        for j in range(len(k)):
            if vis[i][j]:
                s = 0.0
                for t in range(d):
                    s += q[i][t] * k[j][t]
                scores.append((j, scale * s))
        if not scores:
            out.append([0.0] * d)
            lse.append(-math.inf)
            continue
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        out.append([sum(x * v[j][t] for j, x in w) / tot for t in range(d)])
        lse.append(mx + math.log(tot))
    return out, lse


@pytest.mark.parametrize("key", sorted(LITERAL_4x4, key=str))
def test_bruteforce_4x4_literal_tables(key):
    causal, window, Lq, Lk = key
    table = np.array(LITERAL_4x4[key], dtype=bool)
    got = oracle.visible_matrix(np.arange(4), 4, Lq, Lk, causal, window)
    np.testing.assert_array_equal(got, table)
    for i in range(4):
        for j in range(4):
            assert oracle.visible(i, j, Lq, Lk, causal, window) == table[i, j]

    rng = np.random.default_rng(11)
    d = 3
    q = rng.integers(-2, 3, size=(4, d)).astype(np.float64)
    k = rng.integers(-2, 3, size=(4, d)).astype(np.float64)
    v = rng.integers(-3, 4, size=(4, d)).astype(np.float64)
    scale = 0.5
    o, lse = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None],
                              scale=scale, causal=causal, window_left=window,
                              seqlens_q=[Lq], seqlens_k=[Lk])
    eo, el = _scalar_attention(q.tolist(), k.tolist(), v.tolist(), scale, table.tolist())
    np.testing.assert_allclose(o[0, :, 0], np.array(eo), rtol=0, atol=1e-13)
    for a, b in zip(lse[0, 0], el):
        if math.isinf(b):
            assert a == -math.inf
        else:
            assert abs(a - b) < 1e-13


# ---------------------------------------------------------------------------
# P1: Q = 0 -> O is the mean of the visible V rows and LSE = ln(#visible)
# ---------------------------------------------------------------------------
def _closed_form_range(i, Lq, Lk, causal, W):
    """[lo, hi) of visible keys for row i, written from the definitions."""
    if i >= Lq:
        return 0, 0
    pos = i + Lk - Lq
    hi = min(Lk, pos + 1) if causal else Lk
    lo = max(0, pos - W + 1) if W > 0 else 0
    return lo, max(lo, hi)


@pytest.mark.parametrize("causal,W,Lq,Lk,Hq,Hkv", [
    (False, -1, 37, 37, 2, 2), (True, -1, 37, 37, 4, 2), (True, 5, 37, 37, 4, 1),
    (False, 7, 37, 37, 2, 1), (False, -1, 37, 20, 3, 3), (True, -1, 20, 37, 2, 1),
    (True, 9, 37, 29, 6, 2), (True, -1, 37, 0, 2, 2),
])
def test_zero_query_closed_form(causal, W, Lq, Lk, Hq, Hkv):
    Nq, Nk, d = 37, 37, 8
    rng = np.random.default_rng(3)
    q = np.zeros((1, Nq, Hq, d))
    k = rng.standard_normal((1, Nk, Hkv, d))
    # distinct V per kv head so that a wrong GQA map is visible
    v = rng.standard_normal((1, Nk, Hkv, d)) + 10.0 * np.arange(Hkv)[None, None, :, None]
    o, lse = oracle.attention(q, k, v, scale=0.125, causal=causal, window_left=W,
                              seqlens_q=[Lq], seqlens_k=[Lk])
    G = Hq // Hkv
    for i in range(Nq):
        lo, hi = _closed_form_range(i, Lq, Lk, causal, W)
        for h in range(Hq):
            if hi == lo:
                assert np.all(o[0, i, h] == 0.0)
                assert lse[0, h, i] == -np.inf
            else:
                np.testing.assert_allclose(o[0, i, h], v[0, lo:hi, h // G].mean(axis=0),
                                           rtol=0, atol=1e-12)
                assert abs(lse[0, h, i] - math.log(hi - lo)) < 1e-12


# ---------------------------------------------------------------------------
# P2 / P3 / P4: identical V rows, identical K rows, single visible key
# ---------------------------------------------------------------------------
def test_identical_v_rows_return_that_row():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 33, 4, 16))
    k = rng.standard_normal((2, 33, 2, 16))
    row = rng.standard_normal(16)
    v = np.broadcast_to(row, (2, 33, 2, 16)).copy()
    o, _ = oracle.attention(q, k, v, scale=0.25, causal=True, window_left=6,
                            seqlens_k=[33, 21])
    # every non-empty row returns the common V row
    _, lse = oracle.attention(q, k, v, scale=0.25, causal=True, window_left=6,
                              seqlens_k=[33, 21])
    nonempty = np.isfinite(lse).transpose(0, 2, 1)       # [B, N, H]
    np.testing.assert_allclose(o[nonempty], np.broadcast_to(row, o[nonempty].shape),
                               rtol=0, atol=1e-12)


def test_identical_k_rows_give_visible_mean_any_q():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 40, 2, 8)) * 3
    krow = rng.standard_normal(8)
    k = np.broadcast_to(krow, (1, 40, 2, 8)).copy()
    v = rng.standard_normal((1, 40, 2, 8))
    scale = 0.3
    o, lse = oracle.attention(q, k, v, scale=scale, causal=True, window_left=11)
    for i in range(40):
        lo, hi = _closed_form_range(i, 40, 40, True, 11)
        for h in range(2):
            np.testing.assert_allclose(o[0, i, h], v[0, lo:hi, h].mean(axis=0), atol=1e-12)
            expect = float(np.float32(scale)) * float(q[0, i, h] @ krow) + math.log(hi - lo)
            assert abs(lse[0, h, i] - expect) < 1e-11


def test_causal_row0_is_v0_exactly():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 16, 1, 32))
    k = rng.standard_normal((1, 16, 1, 32))
    v = rng.standard_normal((1, 16, 1, 32))
    o, lse = oracle.attention(q, k, v, scale=0.2, causal=True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert abs(lse[0, 0, 0] - float(np.float32(0.2)) * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14


# ---------------------------------------------------------------------------
# P6 / P7 / P8: shift, permutation and padding invariances
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shift", [0.5, 1000.0])
def test_key_shift_invariance(shift):
    """K -> K + 1 u^T adds scale*q_i.u to every score of row i."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 30, 2, 8))
    k = rng.standard_normal((1, 30, 2, 8))
    v = rng.standard_normal((1, 30, 2, 8))
    u = np.full(8, shift)
    scale = 0.5
    o1, l1 = oracle.attention(q, k, v, scale=scale, causal=True, window_left=9)
    o2, l2 = oracle.attention(q, k + u, v, scale=scale, causal=True, window_left=9)
    assert np.all(np.isfinite(o2))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-9)
    delta = scale * np.einsum("bnhd,d->bhn", q, u)
    np.testing.assert_allclose(l2, l1 + delta, rtol=1e-12, atol=1e-9)


def test_joint_key_permutation_invariance():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 19, 4, 8))
    k = rng.standard_normal((2, 23, 2, 8))
    v = rng.standard_normal((2, 23, 2, 8))
    perm = rng.permutation(23)
    o1, l1 = oracle.attention(q, k, v, scale=0.4)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm], scale=0.4)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


def test_padding_equivalence_with_poison():
    p = workloads.make_prefill(21, 3, 50, 50, 4, 2, 16, "bf16", causal=True,
                               seqlens_k_range=(1, 50), seqlens_q_equal_k=True,
                               poison_padding=True)
    q, k, v = _f64(p)
    o, lse = oracle.attention(q, k, v, scale=p.scale, causal=True,
                              seqlens_q=p.seqlens_q, seqlens_k=p.seqlens_k)
    for b in range(3):
        L = int(p.seqlens_k[b])
        o_ref, l_ref = oracle.attention(q[b:b + 1, :L], k[b:b + 1, :L], v[b:b + 1, :L],
                                        scale=p.scale, causal=True)
        np.testing.assert_allclose(o[b, :L], o_ref[0], atol=1e-12)
        np.testing.assert_allclose(lse[b, :, :L], l_ref[0], atol=1e-12)
        assert np.all(o[b, L:] == 0.0) and np.all(lse[b, :, L:] == -np.inf)


# ---------------------------------------------------------------------------
# P9: library cross-check (torch SDPA in float64, scipy logsumexp)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal,W,seq", [(False, -1, False), (True, -1, False),
                                           (True, 64, False), (False, -1, True),
                                           (True, 100, True)])
def test_matches_torch_sdpa_and_scipy_logsumexp(causal, W, seq):
    p = workloads.make_prefill(31, 2, 150, 150, 6, 3, 32, "bf16", causal=causal,
                               window_left=W, seqlens_k_range=(90, 150) if seq else None)
    q, k, v = _f64(p)
    o, lse = oracle.attention(q, k, v, scale=p.scale, causal=causal, window_left=W,
                              seqlens_k=p.seqlens_k)
    B, N, Hq, d = q.shape
    G = Hq // k.shape[2]
    for b in range(B):
        Lk = N if p.seqlens_k is None else int(p.seqlens_k[b])
        # mask written independently from the definitions, as torch booleans
        i = torch.arange(N)[:, None]
        j = torch.arange(N)[None, :]
        pos = i + (Lk - N)
        mask = (j < Lk) & (i >= 0)                               # [N, N]
        if causal:
            mask = mask & (j <= pos)
        if W > 0:
            mask = mask & (j > pos - W)
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)                      # [H, N, d]
        kt = torch.from_numpy(k[b]).permute(1, 0, 2).repeat_interleave(G, 0)
        vt = torch.from_numpy(v[b]).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=float(np.float32(p.scale)))
        rows = mask.any(dim=1).numpy()
        np.testing.assert_allclose(o[b][rows], ref.permute(1, 0, 2).numpy()[rows],
                                   rtol=0, atol=1e-12)
        s = float(np.float32(p.scale)) * torch.einsum("hnd,hmd->hnm", qt, kt).numpy()
        s = np.where(mask.numpy()[None], s, -np.inf)
        ref_lse = scipy.special.logsumexp(s, axis=-1)
        np.testing.assert_allclose(lse[b][:, rows], ref_lse[:, rows], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P10: the blockwise online recurrence and the split-KV combine rule reach
# the three-step result (fp64)
# ---------------------------------------------------------------------------
def _online(qr, k, v, scale, vis, block):
    n, d = qr.shape
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, d))
    for j0 in range(0, k.shape[0], block):
        s = scale * (qr @ k[j0:j0 + block].T)
        s = np.where(vis[:, j0:j0 + block], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - ref)
        pblk = np.exp(s - ref[:, None])
        l = alpha * l + pblk.sum(axis=1)
        acc = alpha[:, None] * acc + pblk @ v[j0:j0 + block]
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(l[:, None] > 0, acc / l[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return o, lse


@pytest.mark.parametrize("block", [1, 7, 64, 128, 300])
def test_online_recurrence_matches_three_step(block):
    rng = np.random.default_rng(12)
    N, d = 300, 16
    q = rng.standard_normal((N, d)) * 2
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    scale = 0.25
    vis = oracle.visible_matrix(np.arange(N), N, 290, 271, True, 50)
    o_ref, l_ref = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None],
                                    scale=scale, causal=True, window_left=50,
                                    seqlens_q=[290], seqlens_k=[271])
    o, lse = _online(q, k, v, float(np.float32(scale)), vis, block)
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=0, atol=1e-12)
    fin = np.isfinite(l_ref[0, 0])
    np.testing.assert_array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], l_ref[0, 0][fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 33, 256, 1000])
def test_split_kv_combine_matches_decode(chunk):
    """Partial (O~, m, l) per key chunk, merged by max/exp-weighted sums."""
    prob = workloads.make_decode(41, 3, 8, 2, 16, 700, (1, 700), "f32")
    q = workloads.to_f64(prob.q, "f32")
    kc = workloads.to_f64(prob.k_cache, "f32")
    vc = workloads.to_f64(prob.v_cache, "f32")
    o_ref, l_ref = oracle.decode(q, kc, vc, prob.seqlens_k, scale=prob.scale)
    sc = float(np.float32(prob.scale))
    for b in range(3):
        L = int(prob.seqlens_k[b])
        for h in range(8):
            parts = []
            for c0 in range(0, L, chunk):
                s = sc * (kc[b, c0:c0 + chunk][:L - c0, h // 4] @ q[b, h])
                m = s.max()
                p = np.exp(s - m)
                parts.append((m, p.sum(), p @ vc[b, c0:c0 + chunk][:L - c0, h // 4]))
            M = max(m for m, _, _ in parts)
            Lsum = sum(np.exp(m - M) * l for m, l, _ in parts)
            O = sum(np.exp(m - M) * ot for m, _, ot in parts) / Lsum
            np.testing.assert_allclose(O, o_ref[b, h], atol=1e-12)
            assert abs(M + math.log(Lsum) - l_ref[b, h]) < 1e-12


# ---------------------------------------------------------------------------
# Decode-specific pins
# ---------------------------------------------------------------------------
def test_decode_closed_forms_and_poison():
    prob = workloads.make_decode(42, 4, 4, 2, 8, 64, (1, 64), "bf16",
                                 lengths=np.array([1, 17, 64, 0], dtype=np.int32))
    q = np.zeros((4, 4, 8))
    kc = workloads.to_f64(prob.k_cache, "bf16")
    vc = workloads.to_f64(prob.v_cache, "bf16")
    assert np.isnan(kc[0, 1:]).all()                 # poisoned tail is present
    o, lse = oracle.decode(q, kc, vc, prob.seqlens_k, scale=prob.scale)
    for b, L in enumerate([1, 17, 64, 0]):
        for h in range(4):
            if L == 0:
                assert np.all(o[b, h] == 0) and lse[b, h] == -np.inf
                continue
            np.testing.assert_allclose(o[b, h], vc[b, :L, h // 2].mean(axis=0), atol=1e-12)
            assert abs(lse[b, h] - math.log(L)) < 1e-12
    # L = 1 returns V[0] exactly for any query
    qr = workloads.to_f64(prob.q, "bf16")
    o1, _ = oracle.decode(qr, kc, vc, prob.seqlens_k, scale=prob.scale)
    assert np.array_equal(o1[0, 1], vc[0, 0, 0])
    # window W keeps the last W keys
    o2, l2 = oracle.decode(q, kc, vc, prob.seqlens_k, scale=prob.scale, window_left=5)
    np.testing.assert_allclose(o2[2, 0], vc[2, 59:64, 0].mean(axis=0), atol=1e-12)
    assert abs(l2[2, 0] - math.log(5)) < 1e-12


# ---------------------------------------------------------------------------
# Hand-derived fixtures (closed forms with their derivations)
# ---------------------------------------------------------------------------
def test_golden_closed_forms():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 3
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        o, lse = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None],
                                  scale=c["scale"], causal=c["causal"],
                                  window_left=c.get("window_left", -1))
        np.testing.assert_allclose(o[0, :, 0], np.array(c["expect_o"]), rtol=0,
                                   atol=1e-12, err_msg=c["name"])
        exp_lse = [(-math.inf if x is None else x) for x in c["expect_lse"]]
        np.testing.assert_allclose(lse[0, 0], exp_lse, rtol=0, atol=1e-12,
                                   err_msg=c["name"])


# ---------------------------------------------------------------------------
# Input generator: bf16 rounding and determinism
# ---------------------------------------------------------------------------
def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65504.0, 1e-40],
                    dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(vals)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80 and bits[2] == 0x3F82
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 100
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(workloads.f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(workloads.bf16_bits_to_f32(ref),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_generator_hashes_are_stable():
    with open(os.path.join(GOLDEN, "input_hashes.json")) as f:
        stored = json.load(f)
    p = workloads.make_workload(1)
    assert p.sha256() == stored["workload_1"]
    small = workloads.make_prefill(5, 2, 70, 70, 4, 2, 64, "bf16", causal=True,
                                   seqlens_k_range=(1, 70))
    assert small.sha256() == stored["prefill_small"]
    dec = workloads.make_decode(6, 3, 4, 2, 64, 300, (1, 300), "bf16")
    assert dec.sha256() == stored["decode_small"]
    pdec = workloads.make_decode_paged(6, 3, 4, 2, 64, 300, (1, 300), 16, "bf16")
    assert pdec.sha256() == stored["decode_paged_small"]
    fdec = workloads.make_decode(6, 3, 4, 2, 64, 300, (1, 300), "bf16", kv_dtype="fp8_e4m3")
    assert fdec.sha256() == stored["decode_fp8_small"]


def test_nan_on_visible_key_propagates():
    """Only a row with no visible key is 'empty'; NaN data must not look empty."""
    q = np.ones((1, 3, 1, 2))
    k = np.zeros((1, 3, 1, 2))
    v = np.ones((1, 3, 1, 2))
    k[0, 1, 0, 0] = np.nan
    o, lse = oracle.attention(q, k, v, scale=1.0, causal=True)
    assert np.all(o[0, 0, 0] == 1.0) and lse[0, 0, 0] == math.log(1.0)
    assert np.all(np.isnan(o[0, 1:, 0])) and np.all(np.isnan(lse[0, 0, 1:]))


# ---------------------------------------------------------------------------
# ALiBi bias (ops-transformer practice page, section 三: after QK^T/sqrt(d)
# every pair (i, j) gets -m * |i - j|, m a per-head slope)
# ---------------------------------------------------------------------------
def test_alibi_tiny_exact_fractions():
    """Q = 0 makes every score 0, so with slope ln 2 the weights of row i are
    2^-|i-j|.  With V the identity (one-hot per key) row i of O is exactly
    those weights normalised: row 0 of a 4-key non-causal problem is
    (1, 1/2, 1/4, 1/8) / (15/8) = (8, 4, 2, 1) / 15, row 1 is
    (1/2, 1, 1/2, 1/4) / (9/4) = (2, 4, 2, 1) / 9."""
    q = np.zeros((1, 4, 1, 4))
    k = np.zeros((1, 4, 1, 4))
    v = np.eye(4)[None, :, None, :]
    o, lse = oracle.attention(q, k, v, scale=1.0, alibi_slopes=[math.log(2)])
    ln2 = float(np.float32(math.log(2)))        # slopes pass through float32
    w = np.exp2(-np.abs(np.arange(4)[:, None] - np.arange(4)[None, :]) * ln2 / math.log(2))
    np.testing.assert_allclose(o[0, 0, 0], np.array([8, 4, 2, 1]) / 15, rtol=1e-6)
    np.testing.assert_allclose(o[0, 1, 0], np.array([2, 4, 2, 1]) / 9, rtol=1e-6)
    np.testing.assert_allclose(o[0, :, 0], w / w.sum(axis=1, keepdims=True), rtol=1e-12)
    # LSE of row 0 = ln(15/8) up to the float32 rounding of the slope
    assert abs(lse[0, 0, 0] - math.log(15 / 8)) < 1e-6


def test_alibi_causal_geometric_closed_form():
    """Q = 0, causal, slope m, V = key index: row i averages j <= i with
    weights r^(i-j), r = e^-m.  With S0 = sum_t r^t and S1 = sum_t t r^t over
    t = 0..i (geometric series in closed form), O_i = i - S1/S0 and
    LSE_i = ln S0."""
    N, m = 50, 0.3
    q = np.zeros((1, N, 1, 2))
    k = np.zeros((1, N, 1, 2))
    v = np.zeros((1, N, 1, 2))
    v[0, :, 0, 0] = np.arange(N)
    o, lse = oracle.attention(q, k, v, scale=1.0, causal=True, alibi_slopes=[m])
    r = math.exp(-float(np.float32(m)))
    for i in (0, 1, 7, N - 1):
        S0 = (1 - r ** (i + 1)) / (1 - r)
        S1 = r * (1 - (i + 1) * r ** i + i * r ** (i + 1)) / (1 - r) ** 2
        assert abs(o[0, i, 0, 0] - (i - S1 / S0)) < 1e-10
        assert abs(lse[0, 0, i] - math.log(S0)) < 1e-10


def test_alibi_symmetry_and_limits():
    """Non-causal with Q = 0 and V = key index: the middle row of an odd
    length sees a symmetric weight profile, so O = its own index.  A huge
    slope makes each row copy the value of the key at its own position (the
    only key at distance 0), in both alignments (Lq = Lk and Lq < Lk)."""
    N = 41
    q = np.zeros((1, N, 1, 2))
    k = np.zeros((1, N, 1, 2))
    v = np.zeros((1, N, 1, 2))
    v[0, :, 0, 0] = np.arange(N)
    o, _ = oracle.attention(q, k, v, scale=1.0, alibi_slopes=[0.7])
    assert abs(o[0, N // 2, 0, 0] - N // 2) < 1e-12
    rng = np.random.default_rng(3)
    qr = rng.standard_normal((1, 10, 2, 8))
    kr = rng.standard_normal((1, 30, 2, 8))
    vr = rng.standard_normal((1, 30, 2, 8))
    o, _ = oracle.attention(qr, kr, vr, scale=0.3, causal=True, alibi_slopes=[80.0, 90.0])
    # query row i sits at key position i + 20 (bottom-right alignment)
    np.testing.assert_allclose(o[0, :, :, :], vr[0, 20:30], atol=1e-12)


def test_alibi_zero_slopes_and_decode_consistency():
    """Zero slopes change nothing; decode with ALiBi equals the last row of the
    prefill of the same sequence, whose query sits at position L - 1."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 9, 4, 16))
    k = rng.standard_normal((2, 9, 2, 16))
    v = rng.standard_normal((2, 9, 2, 16))
    o0, l0 = oracle.attention(q, k, v, scale=0.25, causal=True)
    o1, l1 = oracle.attention(q, k, v, scale=0.25, causal=True, alibi_slopes=[0.0] * 4)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    slopes = [0.5, 0.25, 0.125, 0.0625]
    op, lp = oracle.attention(q, k, v, scale=0.25, causal=True, alibi_slopes=slopes)
    od, ld = oracle.decode(q[:, -1], k, v, [9, 9], scale=0.25, alibi_slopes=slopes)
    np.testing.assert_allclose(od, op[:, -1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ld, lp[:, :, -1], rtol=1e-12, atol=1e-12)


def test_alibi_matches_torch_sdpa_float_mask():
    """Library cross-check: torch's scaled_dot_product_attention (fp64, CPU)
    with the bias passed as an additive float mask (the causal part as -inf)."""
    rng = np.random.default_rng(5)
    B, N, H, d = 2, 33, 3, 16
    q = rng.standard_normal((B, N, H, d))
    k = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    slopes = np.float32([0.3, 0.05, 1.5]).astype(np.float64)
    o, _ = oracle.attention(q, k, v, scale=d ** -0.5, causal=True, alibi_slopes=slopes)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    bias = -slopes[:, None, None] * np.abs(i - j)[None]
    bias = np.where(j <= i, bias, -np.inf)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(bias)[None], scale=d ** -0.5)
    np.testing.assert_allclose(o, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Paged KV cache: the gather and decode over it
# ---------------------------------------------------------------------------
def test_gather_paged_literal():
    """Page p, slot s of this pool holds 2p + s; the rows are read off by hand."""
    pool = np.arange(8).reshape(4, 2)
    assert oracle.gather_paged(pool, [2, 0, 3], 5).tolist() == [4, 5, 0, 1, 6]
    assert oracle.gather_paged(pool, [3, 1], 4).tolist() == [6, 7, 2, 3]
    assert oracle.gather_paged(pool, [1], 0).shape == (0,)


def _scatter_pages(cache, lengths, P, seed):
    """Inverse of the gather, written independently of the oracle: each
    sequence's rows go page by page into shuffled physical pages; unused
    slots, the spare page and every table entry past the used pages are NaN."""
    B, cap = cache.shape[:2]
    per = -(-cap // P)
    used = [-(-int(L) // P) for L in lengths]
    n_pages = sum(used) + 1
    order = np.random.default_rng(seed).permutation(n_pages)
    pool = np.full((n_pages, P) + cache.shape[2:], np.nan)
    table = np.full((B, per), order[-1], dtype=np.int64)
    nxt = 0
    for b in range(B):
        for pg in range(used[b]):
            phys = order[nxt]
            nxt += 1
            table[b, pg] = phys
            rows = cache[b, pg * P:min(int(lengths[b]), (pg + 1) * P)]
            pool[phys, :len(rows)] = rows
    return pool, table


@pytest.mark.parametrize("P", [1, 3, 16])
@pytest.mark.parametrize("window", [-1, 5])
def test_paged_decode_equals_contiguous(P, window):
    """Same logical rows in a shuffled pool: the same result, bit for bit."""
    prob = workloads.make_decode(43, 4, 8, 2, 16, 96, (0, 96), "bf16",
                                 lengths=np.array([1, 17, 96, 0], dtype=np.int32))
    q = workloads.to_f64(prob.q, "bf16")
    kc = workloads.to_f64(prob.k_cache, "bf16")
    vc = workloads.to_f64(prob.v_cache, "bf16")
    slopes = np.linspace(0.05, 0.4, 8).astype(np.float32)
    kp, table = _scatter_pages(kc, prob.seqlens_k, P, seed=P)
    vp, table2 = _scatter_pages(vc, prob.seqlens_k, P, seed=P)
    assert np.array_equal(table, table2)
    for sl in (None, slopes):
        o_ref, l_ref = oracle.decode(q, kc, vc, prob.seqlens_k, scale=prob.scale,
                                     window_left=window, alibi_slopes=sl)
        o, l = oracle.decode_paged(q, kp, vp, table, prob.seqlens_k, scale=prob.scale,
                                   window_left=window, alibi_slopes=sl)
        assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref)
        assert np.isfinite(o).all()


def test_paged_decode_zero_query_mean_of_gathered_rows():
    """q = 0: O is the mean of the gathered V rows, LSE = ln L (hand-checked rows)."""
    vp = np.zeros((3, 2, 1, 1))
    vp[:, :, 0, 0] = [[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]]
    kp = np.ones_like(vp)
    q = np.zeros((1, 1, 1))
    table = np.array([[2, 0]])
    o, l = oracle.decode_paged(q, kp, vp, table, [3], scale=1.0)
    assert o[0, 0, 0] == pytest.approx((100.0 + 200.0 + 1.0) / 3, abs=1e-12)
    assert l[0, 0] == pytest.approx(math.log(3), abs=1e-12)
    # lengths clamp to the table's capacity (2 pages x 2 slots)
    o, l = oracle.decode_paged(q, kp, vp, table, [9], scale=1.0)
    assert o[0, 0, 0] == pytest.approx((100.0 + 200.0 + 1.0 + 2.0) / 4, abs=1e-12)


def test_paged_generator_holds_the_contiguous_rows():
    """The paged generator and the contiguous one hold the same logical cache."""
    a = workloads.make_decode(44, 3, 4, 2, 8, 100, (1, 100), "bf16")
    p = workloads.make_decode_paged(44, 3, 4, 2, 8, 100, (1, 100), 16, "bf16")
    assert np.array_equal(a.q, p.q) and np.array_equal(a.seqlens_k, p.seqlens_k)
    for b in range(3):
        L = int(a.seqlens_k[b])
        assert np.array_equal(oracle.gather_paged(p.k_pool, p.block_table[b], L), a.k_cache[b, :L])
        assert np.array_equal(oracle.gather_paged(p.v_pool, p.block_table[b], L), a.v_cache[b, :L])
    # every table entry past the used pages names a NaN page
    for b in range(3):
        used = -(-int(p.seqlens_k[b]) // 16)
        for e in p.block_table[b, used:]:
            assert (p.k_pool[e] == workloads.BF16_QNAN).all()


# ---------------------------------------------------------------------------
# FP8 E4M3 KV cache: code values and dequantized decode
# ---------------------------------------------------------------------------
# code -> value, read off the E4M3FN bit layout by hand
E4M3_LITERALS = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
    0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x47: 3.75, 0x77: 240.0, 0x78: 256.0,
    0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0,
}


def test_fp8_e4m3_literal_codes():
    for code, val in E4M3_LITERALS.items():
        got = oracle.fp8_e4m3_value(np.array([code], dtype=np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), hex(code)
    nan = oracle.fp8_e4m3_value(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(nan).all()


def test_fp8_e4m3_all_codes_match_torch_and_order():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], ref[fin])
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)                    # 0x00 .. 0x7E strictly increasing
    assert np.array_equal(ours[0x80:0xFF], -pos)       # the sign bit only negates


def test_dequantized_decode_scaling_laws():
    """A K scale multiplies every score (the same as scaling softmax_scale);
    a V scale multiplies O and leaves LSE alone; constant K codes give the
    mean of the dequantized V rows."""
    prob = workloads.make_decode(45, 3, 8, 2, 16, 80, (1, 80), "bf16", kv_dtype="fp8_e4m3")
    q = workloads.to_f64(prob.q, "bf16")
    ks, vs = prob.k_scale, prob.v_scale
    k = oracle.dequantize_kv(prob.k_cache, ks)
    v = oracle.dequantize_kv(prob.v_cache, vs)
    o1, l1 = oracle.decode(q, k, v, prob.seqlens_k, scale=0.25)
    o2, l2 = oracle.decode(q, oracle.dequantize_kv(prob.k_cache, 2 * ks), v, prob.seqlens_k,
                           scale=0.125)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
    o3, l3 = oracle.decode(q, k, oracle.dequantize_kv(prob.v_cache, 2 * vs), prob.seqlens_k,
                           scale=0.25)
    np.testing.assert_allclose(o3, 2 * o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, l1, rtol=0, atol=0)
    const = np.where(prob.k_cache == workloads.FP8_E4M3_QNAN, prob.k_cache, np.uint8(0x38))
    o4, l4 = oracle.decode(q, oracle.dequantize_kv(const, ks), v, prob.seqlens_k, scale=0.25)
    for b in range(3):
        L = int(prob.seqlens_k[b])
        for h in range(8):
            np.testing.assert_allclose(o4[b, h], v[b, :L, h // 4].mean(axis=0), atol=1e-12)
            assert abs(l4[b, h] - (0.25 * float(ks[h // 4]) * q[b, h].sum() + math.log(L))) < 1e-12


def test_fp8_generator_codes_round_to_nearest():
    """The generator's codes hold the drawn values to E4M3's half-step, and
    each head's largest magnitude lands on +-448."""
    prob = workloads.make_decode(46, 2, 4, 2, 16, 64, (64, 64), "bf16", kv_dtype="fp8_e4m3")
    raw = workloads.make_decode(46, 2, 4, 2, 16, 64, (64, 64), "f32")
    for codes, sc, x in ((prob.k_cache, prob.k_scale, raw.k_cache),
                         (prob.v_cache, prob.v_scale, raw.v_cache)):
        vals = oracle.fp8_e4m3_value(codes)
        y = x.astype(np.float64) / sc.astype(np.float64)[:, None]
        # E4M3 step at |y|: 2^(floor(log2 |y|) - 3), at least the subnormal step 2^-9
        step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))), -6) - 3)
        assert np.all(np.abs(vals - y) <= 0.5 * step * (1 + 1e-6))
        for h in range(2):
            assert np.abs(vals[:, :, h]).max() == 448.0


# ---------------------------------------------------------------------------
# RoPE: pair rotation and its use in attention
# ---------------------------------------------------------------------------
def _angle_tables(n_pos, half, base=10000.0, dtype=np.float32):
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / (2 * half))
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def test_rope_literal_rotation():
    # pair 0 turned by 90 degrees, pair 1 by 180 degrees (exact table values)
    cos_t = np.array([[0.0, -1.0]], np.float32)
    sin_t = np.array([[1.0, 0.0]], np.float32)
    out = oracle.rope_rotate(np.array([[1.0, 0.0, 0.0, 1.0]]), [0], cos_t, sin_t, 4)
    assert out.tolist() == [[0.0, 1.0, 0.0, -1.0]]
    # rotary_dim 2 leaves the second pair alone
    out = oracle.rope_rotate(np.array([[1.0, 0.0, 0.0, 1.0]]), [0], cos_t, sin_t, 2)
    assert out.tolist() == [[0.0, 1.0, 0.0, 1.0]]


def test_rope_matches_complex_multiplication_and_keeps_pair_norms():
    rng = np.random.default_rng(7)
    cos_t, sin_t = _angle_tables(50, 8)
    x = rng.standard_normal((20, 24))
    pos = rng.integers(0, 50, 20)
    out = oracle.rope_rotate(x, pos, cos_t, sin_t, 16)
    z = (x[:, 0:16:2] + 1j * x[:, 1:16:2]) * (cos_t[pos].astype(np.float64) + 1j * sin_t[pos].astype(np.float64))
    np.testing.assert_allclose(out[:, 0:16:2], z.real, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[:, 1:16:2], z.imag, rtol=0, atol=1e-14)
    assert np.array_equal(out[:, 16:], x[:, 16:])
    n_in = x[:, 0:16:2] ** 2 + x[:, 1:16:2] ** 2
    n_out = out[:, 0:16:2] ** 2 + out[:, 1:16:2] ** 2
    c64, s64 = cos_t[pos].astype(np.float64), sin_t[pos].astype(np.float64)
    np.testing.assert_allclose(n_out, n_in * (c64 ** 2 + s64 ** 2), rtol=1e-12)


def test_rope_scores_depend_on_relative_position():
    """With angles proportional to the position, q at m against k at n gives
    the same product as q at m + t against k at n + t (to the float32
    rounding of the table entries, which the oracle reads as float32)."""
    rng = np.random.default_rng(8)
    cos_t, sin_t = _angle_tables(400, 16)
    q, k = rng.standard_normal((1, 32)), rng.standard_normal((1, 32))
    for m, n, t in ((5, 3, 100), (0, 0, 399), (250, 10, 37)):
        a = oracle.rope_rotate(q, [m], cos_t, sin_t, 32) @ oracle.rope_rotate(k, [n], cos_t, sin_t, 32).T
        b = oracle.rope_rotate(q, [m + t], cos_t, sin_t, 32) @ oracle.rope_rotate(k, [n + t], cos_t, sin_t, 32).T
        assert abs(a - b) < 2e-6 * (1 + abs(a))


def test_rope_attention_query_alignment():
    """The last M query rows of an N-row causal problem are the same rows as a
    problem holding only those M queries against the same N keys (query row
    i sits at position i + Lk - Lq), so RoPE must give them the same output."""
    p = workloads.make_prefill(80, 1, 40, 40, 2, 1, 16, "f32", causal=True)
    q, k, v = _f64(p)
    cos_t, sin_t = _angle_tables(40, 6)
    rope = (cos_t, sin_t, 12)
    o_full, l_full = oracle.attention(q, k, v, scale=0.3, causal=True, rope=rope)
    o_tail, l_tail = oracle.attention(q[:, 30:], k, v, scale=0.3, causal=True, rope=rope)
    np.testing.assert_allclose(o_tail, o_full[:, 30:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_tail, l_full[:, :, 30:], rtol=0, atol=1e-13)
    # and rotation really changes the result (it is not a no-op)
    o_plain, _ = oracle.attention(q, k, v, scale=0.3, causal=True)
    assert np.abs(o_plain - o_full).max() > 1e-3


def test_rope_decode_query_at_last_position():
    """Decode rotates the query at L - 1 and reads keys as stored: against
    keys rotated at their positions, it equals one-row causal attention with
    RoPE on both sides."""
    dp = workloads.make_decode(81, 3, 4, 2, 16, 30, (1, 30), "f32",
                               lengths=np.array([30, 7, 1], dtype=np.int32))
    q = workloads.to_f64(dp.q, "f32")
    kc = workloads.to_f64(dp.k_cache, "f32")
    vc = workloads.to_f64(dp.v_cache, "f32")
    cos_t, sin_t = _angle_tables(30, 8)
    rope = (cos_t, sin_t, 16)
    k_rot = kc.copy()
    for b in range(3):
        L = int(dp.seqlens_k[b])
        for h in range(2):
            k_rot[b, :L, h] = oracle.rope_rotate(kc[b, :L, h], np.arange(L), *rope)
    o, l = oracle.decode(q, k_rot, vc, dp.seqlens_k, scale=0.25, rope_q=rope)
    for b in range(3):
        L = int(dp.seqlens_k[b])
        ro, rl = oracle.attention(q[b][None, None], kc[b, :L][None], vc[b, :L][None], scale=0.25,
                                  causal=True, rope=rope)
        np.testing.assert_allclose(o[b], ro[0, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[b], rl[0, :, 0], rtol=0, atol=1e-13)


def test_rope_rejects_positions_outside_the_tables():
    cos_t, sin_t = _angle_tables(10, 4)
    x = np.ones((2, 8))
    with pytest.raises(ValueError):
        oracle.rope_rotate(x, [-1, 3], cos_t, sin_t, 8)
    with pytest.raises(ValueError):
        oracle.rope_rotate(x, [0, 10], cos_t, sin_t, 8)
    oracle.rope_rotate(x, [0, 9], cos_t, sin_t, 8)


def _rotate_complex(x, pos, cos_t, sin_t, rdim):
    """Independent coding of the pair rotation: complex multiplication."""
    x = np.array(x, dtype=np.float64)
    z = (x[:, 0:rdim:2] + 1j * x[:, 1:rdim:2]) * (
        cos_t[pos, :rdim // 2].astype(np.float64) + 1j * sin_t[pos, :rdim // 2].astype(np.float64))
    x[:, 0:rdim:2], x[:, 1:rdim:2] = z.real, z.imag
    return x


@pytest.mark.parametrize("causal", [False, True])
def test_rope_more_queries_than_keys(causal):
    """Lq > Lk: query row i sits at i + Lk - Lq; the first Lq - Lk rows have
    no position in the tables and see nothing under RoPE (causal: they are
    empty anyway).  The other rows match the scalar loop over inputs rotated
    by complex multiplication.  Static extents (Nq 6, Nk 3) and valid lengths
    (seqlens_k 2 and 6 of 6) both."""
    rng = np.random.default_rng(90)
    cos_t, sin_t = _angle_tables(8, 4)
    rope = (cos_t, sin_t, 8)
    for Nq, Nk, lens in ((6, 3, None), (6, 6, [2, 6])):
        B = 1 if lens is None else 2
        q = rng.integers(-3, 4, (B, Nq, 1, 8)).astype(np.float64)
        k = rng.integers(-3, 4, (B, Nk, 1, 8)).astype(np.float64)
        v = rng.integers(-3, 4, (B, Nk, 1, 8)).astype(np.float64)
        o, l = oracle.attention(q, k, v, scale=0.25, causal=causal, rope=rope, seqlens_k=lens)
        for b in range(B):
            Lk = Nk if lens is None else lens[b]
            off = Lk - Nq
            first = max(0, -off)                      # rows before position 0
            qr = _rotate_complex(q[b, first:, 0], np.arange(first, Nq) + off, cos_t, sin_t, 8)
            kr = _rotate_complex(k[b, :Lk, 0], np.arange(Lk), cos_t, sin_t, 8)
            vis = [[(not causal) or j <= i + off for j in range(Lk)] for i in range(first, Nq)]
            so, sl = _scalar_attention(qr.tolist(), kr.tolist(), v[b, :Lk, 0].tolist(), 0.25, vis)
            assert np.all(o[b, :first, 0] == 0.0) and np.all(l[b, 0, :first] == -np.inf)
            np.testing.assert_allclose(o[b, first:, 0], np.array(so), rtol=0, atol=1e-12)
            np.testing.assert_allclose(l[b, 0, first:], np.array(sl), rtol=0, atol=1e-12)


def test_round_to_dtype_single_rounding_to_nearest_even():
    # ties go to the even neighbour; a value just above a tie goes up, which
    # rounding through fp32 first (double rounding) would get wrong
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40,
                     -(1.0 + 2.0 ** -8 + 2.0 ** -40), 0.0, 3.0])
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 0.0, 3.0])
    assert np.array_equal(oracle.round_to_dtype(vals, "bf16"), want)
    x = np.random.default_rng(3).standard_normal(50000).astype(np.float32) * 30
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.round_to_dtype(x.astype(np.float64), "bf16"), ref)
    y = np.random.default_rng(4).standard_normal(1000)
    assert np.array_equal(oracle.round_to_dtype(y, "f32"), y.astype(np.float32).astype(np.float64))
    # half: against torch's float16 cast of fp32 values, and a tie going to even
    xh = np.random.default_rng(6).standard_normal(50000).astype(np.float32) * 30
    refh = torch.from_numpy(xh).to(torch.float16).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.round_to_dtype(xh.astype(np.float64), "f16"), refh)
    assert oracle.round_to_dtype(np.array([1.0 + 2.0 ** -11]), "f16")[0] == 1.0
    assert np.array_equal(oracle.round_to_dtype(y, None), y)


# ---------------------------------------------------------------------------
# Explicit additive mask
# ---------------------------------------------------------------------------
def test_mask_zero_and_padding_equivalences():
    """A zero mask changes nothing; a key-padding mask of -inf (shape
    [B, 1, 1, Nk], the BERT page's layout) equals valid key lengths."""
    p = workloads.make_prefill(82, 3, 40, 40, 4, 2, 16, "f32")
    q, k, v = _f64(p)
    o0, l0 = oracle.attention(q, k, v, scale=0.3)
    o1, l1 = oracle.attention(q, k, v, scale=0.3, attn_mask=np.zeros((3, 1, 1, 40)))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    lengths = [40, 13, 1]
    pad = np.zeros((3, 1, 1, 40))
    for b, L in enumerate(lengths):
        pad[b, 0, 0, L:] = -np.inf
    o2, l2 = oracle.attention(q, k, v, scale=0.3, attn_mask=pad)
    o3, l3 = oracle.attention(q, k, v, scale=0.3, seqlens_k=lengths)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


def test_mask_as_bias_equals_alibi():
    """A mask holding -m |pos_i - j| gives the ALiBi result (powers of two keep
    both sides exact)."""
    p = workloads.make_prefill(83, 1, 24, 30, 2, 1, 16, "f32", causal=True)
    q, k, v = _f64(p)
    slopes = np.array([0.5, 0.125], np.float32)
    pos = np.arange(24)[:, None] + (30 - 24)
    dist = np.abs(pos - np.arange(30)[None, :]).astype(np.float64)
    mask = -slopes.astype(np.float64)[None, :, None, None] * dist[None, None]
    o1, l1 = oracle.attention(q, k, v, scale=0.25, causal=True, alibi_slopes=slopes)
    o2, l2 = oracle.attention(q, k, v, scale=0.25, causal=True, attn_mask=mask)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_mask_matches_torch_sdpa_float_mask():
    p = workloads.make_prefill(84, 2, 20, 27, 3, 3, 8, "f32")
    q, k, v = _f64(p)
    mask = np.random.default_rng(5).standard_normal((2, 3, 20, 27)) * 3.0
    mask[0, 1, 4, :20] = -np.inf
    o, lse = oracle.attention(q, k, v, scale=0.35, attn_mask=mask)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(k).permute(0, 2, 1, 3),
        torch.from_numpy(v).permute(0, 2, 1, 3), attn_mask=torch.from_numpy(mask),
        scale=float(np.float32(0.35)))            # the scale is an fp32 argument
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
    s = float(np.float32(0.35)) * np.einsum("bqhd,bkhd->bhqk", q, k) + mask
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


def test_half_storage_matches_torch():
    x = np.random.default_rng(9).standard_normal(20000).astype(np.float32) * 50
    bits = workloads._store(x, "f16")
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(workloads.to_f64(bits, "f16"),
                          torch.from_numpy(ref.view(np.int16)).view(torch.float16).double().numpy())
