"""Helpers for the GPU parity tests: device transfer, the library calls, the
oracle calls on the same bits, and the tolerance checks.

Tolerances (element-wise against the fp64 oracle):
* bf16 and half (f16) inputs: max |dO| <= 2e-2 and mean |dO| <= 2e-3 over all of O; these
  are the method's stated bounds.  LSE: max |dLSE| <= 1e-3 -- the scores
  themselves are exact products of bf16 values accumulated in fp32, so LSE
  only carries fp32 rounding (~1e-6 relative); 1e-3 leaves a wide margin
  while still catching a wrong max, sum or log base.
* fp32 inputs: max |dO| <= 1e-4 (the stated bound) and max |dLSE| <= 1e-4.
* rows with no visible key: O exactly 0 and LSE exactly -inf on both sides.
"""
import numpy as np
import torch

import oracle
import transformer_attention_flashattention_amd as fa
import workloads

DEV = torch.device("cuda:0")

TOL = {
    "bf16": dict(max=2e-2, mean=2e-3, lse=1e-3),
    "f16": dict(max=2e-2, mean=2e-3, lse=1e-3),
    "f32": dict(max=1e-4, mean=1e-4, lse=1e-4),
}


def say(msg):
    print(msg, flush=True)


def dev_tensor(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def prefill_inputs(p):
    q, k, v = (dev_tensor(x, p.dtype) for x in (p.q, p.k, p.v))
    sq = torch.from_numpy(p.seqlens_q).to(DEV) if p.seqlens_q is not None else None
    sk = torch.from_numpy(p.seqlens_k).to(DEV) if p.seqlens_k is not None else None
    return q, k, v, sq, sk


def run_prefill(p, **kw):
    q, k, v, sq, sk = prefill_inputs(p)
    o, lse = fa.prefill(q, k, v, causal=p.causal, window=p.window_left, scale=p.scale,
                        seqlens_q=sq, seqlens_k=sk, **kw)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def oracle_prefill(p, rows=None, heads=None, alibi_slopes=None):
    return oracle.attention(workloads.to_f64(p.q, p.dtype), workloads.to_f64(p.k, p.dtype),
                            workloads.to_f64(p.v, p.dtype), scale=p.scale, causal=p.causal,
                            window_left=p.window_left, seqlens_q=p.seqlens_q,
                            seqlens_k=p.seqlens_k, rows=rows, heads=heads,
                            alibi_slopes=alibi_slopes)


def check(o, lse, ro, rl, dtype, ctx=""):
    tol = TOL[dtype]
    assert o.shape == ro.shape, (ctx, o.shape, ro.shape)
    assert lse.shape == rl.shape, (ctx, lse.shape, rl.shape)
    assert np.all(np.isfinite(o)), f"{ctx}: non-finite values in O"
    err = np.abs(o - ro)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin), f"{ctx}: -inf pattern of LSE differs"
    assert np.all(lse[~fin] == -np.inf), f"{ctx}: empty rows must have LSE = -inf"
    lerr = np.abs(lse[fin] - rl[fin]).max() if fin.any() else 0.0
    say(f"  {ctx}: max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} max|dLSE|={lerr:.3e}")
    assert err.max() <= tol["max"], f"{ctx}: max|dO| {err.max():.3e} > {tol['max']}"
    assert err.mean() <= tol["mean"], f"{ctx}: mean|dO| {err.mean():.3e} > {tol['mean']}"
    assert lerr <= tol["lse"], f"{ctx}: max|dLSE| {lerr:.3e} > {tol['lse']}"
    # empty rows: exactly zero output
    empty = ~fin                                   # [B, H, N] or [B, H]
    if empty.any():
        if o.ndim == 4:                            # prefill O is [B, N, H, d]
            assert np.all(o.transpose(0, 2, 1, 3)[empty] == 0.0), f"{ctx}: empty rows not zero"
        else:
            assert np.all(o[empty] == 0.0), f"{ctx}: empty rows not zero"


def decode_inputs(dp):
    q, kc, vc = (dev_tensor(x, dp.dtype) for x in (dp.q, dp.k_cache, dp.v_cache))
    sk = torch.from_numpy(dp.seqlens_k).to(DEV)
    return q, kc, vc, sk


def run_decode(dp, **kw):
    q, kc, vc, sk = decode_inputs(dp)
    o, lse = fa.decode(q, kc, vc, sk, scale=dp.scale, window=dp.window_left, **kw)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def _exact_f32(a, dtype):
    # bf16 / half -> fp32 is exact; the oracle widens each slice it reads to fp64
    if dtype == "bf16":
        return workloads.bf16_bits_to_f32(a)
    if dtype == "f16":
        return np.ascontiguousarray(a).view(np.float16).astype(np.float32)
    return a


def oracle_decode(dp, batches=None, alibi_slopes=None):
    return oracle.decode(workloads.to_f64(dp.q, dp.dtype), _exact_f32(dp.k_cache, dp.dtype),
                         _exact_f32(dp.v_cache, dp.dtype), dp.seqlens_k, scale=dp.scale,
                         window_left=dp.window_left, batches=batches, alibi_slopes=alibi_slopes)


def paged_inputs(pp):
    q, kp, vp = (dev_tensor(x, pp.dtype) for x in (pp.q, pp.k_pool, pp.v_pool))
    sk = torch.from_numpy(pp.seqlens_k).to(DEV)
    table = torch.from_numpy(pp.block_table).to(DEV)
    return q, kp, vp, sk, table


def run_decode_paged(pp, **kw):
    q, kp, vp, sk, table = paged_inputs(pp)
    o, lse = fa.decode(q, kp, vp, sk, scale=pp.scale, window=pp.window_left, block_table=table,
                       **kw)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def oracle_decode_paged(pp, batches=None, alibi_slopes=None, capacity=None):
    seqlens = pp.seqlens_k
    if capacity is not None:
        seqlens = np.minimum(seqlens, capacity)
    return oracle.decode_paged(workloads.to_f64(pp.q, pp.dtype), _exact_f32(pp.k_pool, pp.dtype),
                               _exact_f32(pp.v_pool, pp.dtype), pp.block_table, seqlens,
                               scale=pp.scale, window_left=pp.window_left, batches=batches,
                               alibi_slopes=alibi_slopes)


def fp8_tensor(codes):
    """uint8 E4M3 codes as a torch.float8_e4m3fn device tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(DEV).view(
        torch.float8_e4m3fn)


def run_decode_fp8(dp, **kw):
    q = dev_tensor(dp.q, dp.dtype)
    kc, vc = fp8_tensor(dp.k_cache), fp8_tensor(dp.v_cache)
    sk = torch.from_numpy(dp.seqlens_k).to(DEV)
    o, lse = fa.decode(q, kc, vc, sk, scale=dp.scale, window=dp.window_left,
                       k_scale=torch.from_numpy(dp.k_scale).to(DEV),
                       v_scale=torch.from_numpy(dp.v_scale).to(DEV), **kw)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def oracle_decode_fp8(dp, alibi_slopes=None):
    return oracle.decode(workloads.to_f64(dp.q, dp.dtype),
                         oracle.dequantize_kv(dp.k_cache, dp.k_scale),
                         oracle.dequantize_kv(dp.v_cache, dp.v_scale), dp.seqlens_k,
                         scale=dp.scale, window_left=dp.window_left, alibi_slopes=alibi_slopes)


def run_decode_paged_fp8(pp, **kw):
    q = dev_tensor(pp.q, pp.dtype)
    kp, vp = fp8_tensor(pp.k_pool), fp8_tensor(pp.v_pool)
    sk = torch.from_numpy(pp.seqlens_k).to(DEV)
    table = torch.from_numpy(pp.block_table).to(DEV)
    o, lse = fa.decode(q, kp, vp, sk, scale=pp.scale, window=pp.window_left, block_table=table,
                       k_scale=torch.from_numpy(pp.k_scale).to(DEV),
                       v_scale=torch.from_numpy(pp.v_scale).to(DEV), **kw)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def oracle_decode_paged_fp8(pp, alibi_slopes=None):
    return oracle.decode_paged(workloads.to_f64(pp.q, pp.dtype),
                               oracle.dequantize_kv(pp.k_pool, pp.k_scale),
                               oracle.dequantize_kv(pp.v_pool, pp.v_scale), pp.block_table,
                               pp.seqlens_k, scale=pp.scale, window_left=pp.window_left,
                               alibi_slopes=alibi_slopes)
