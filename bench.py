"""Benchmark of the fused-attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * prefill: causal attention, B=1, 32 heads, N=8192, d=128, bf16
    (the 7B-decoder-shaped workload), one fa_prefill_fwd call;
  * decode: B=64, Hq=32, Hkv=8, d=128, bf16, per-sequence KV lengths drawn
    uniformly in [512, 8192] over a capacity-8192 cache, one fa_decode_fwd
    call (split + combine kernels).
Inputs are generated once (seeded), copied to HBM, and the timed region only
enqueues library calls.  Each call is bracketed by HIP events on the stream
it is launched on (torch's current stream, which the binding passes to the
library), so the per-call averages are kernel time plus launch gaps.

After the timed steps, the same two calls are timed with ALiBi slopes
(reported under "alibi"), and the decode call over the same logical cache
held in a paged pool of 16-row pages in shuffled order (under "paged") and
as FP8 E4M3 codes with per-KV-head scales (under "fp8_kv"), the prefill
with RoPE over all 128 dims (under "rope"), with an explicit [1, 1, 1, N]
additive mask (under "attn_mask"), and in IEEE half (under "f16", same draws
rounded to half; fp16 dense MFMA peak = bf16's); none of these is part of the
step.

Printed: ONE JSON line.  ``value`` is prefill throughput in TFLOP/s on the
algorithmic flop count (only visible (query, key) pairs: 4*d*H*N(N+1)/2);
decode throughput is reported beside it in GB/s on algorithmic bytes (each
valid K and V row read once per GQA group, plus Q, O, LSE, lengths).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 (and fp16) MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def prefill_flops(B, H, N, d):
    return 4.0 * d * H * B * N * (N + 1) / 2.0


def decode_bytes(seqlens, Hq, Hkv, d, elt=2, kv_elt=None):
    kv = float(np.sum(seqlens)) * Hkv * d * (elt if kv_elt is None else kv_elt) * 2
    q_o = 2.0 * len(seqlens) * Hq * d * elt
    return kv + q_o + len(seqlens) * Hq * 4 + len(seqlens) * 4


def measured_traffic(kernels):
    """HBM bytes per launch of the named kernels, from the committed counter
    summary (FETCH_SIZE / WRITE_SIZE scaled by a copy-kernel calibration), or
    None when any of their sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)["kernels"]
        total = 0
        for name in kernels:
            ent = data[name]
            h = hashlib.sha256()
            for src in ent["sources"]:
                with open(os.path.join(ROOT, src), "rb") as f:
                    h.update(f.read())
            if h.hexdigest() != ent["sources_sha256"]:
                return None
            total += ent["traffic_bytes"]
        return total
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timing (used for profiler runs)")
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="heads of the prefill workload the CPU oracle times")
    ap.add_argument("--decode-chunk", type=int, default=0,
                    help="keys per decode split (0 = library choice)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def to_dev(a, dtype, torch, dev):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def cpu_baseline(p, heads):
    """Time the fp64 oracle on a bounded sample of the prefill workload."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    q = workloads.to_f64(p.q[:, :, :heads], "bf16")
    k = workloads.to_f64(p.k[:, :, :heads], "bf16")
    v = workloads.to_f64(p.v[:, :, :heads], "bf16")
    t0 = time.perf_counter()
    oracle.attention(q, k, v, scale=p.scale, causal=True)
    dt = time.perf_counter() - t0
    B, N = p.q.shape[0], p.q.shape[1]
    flops = prefill_flops(B, heads, N, p.q.shape[3])
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 NumPy three-step oracle on {heads} of 32 heads of the causal "
                      f"N=8192 d=128 prefill (all rows), {dt:.2f} s wall, {cpu}, "
                      f"affinity {len(os.sched_getaffinity(0))} cpus"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_attention_flashattention_amd as fa
    import workloads

    fa.load_library()
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}))
        return

    # ---- inputs (seeded, generated once, resident in HBM) ------------------
    p = workloads.make_workload(3)
    B, N, H, d = p.q.shape
    q, k, v = (to_dev(x, "bf16", torch, dev) for x in (p.q, p.k, p.v))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    dp = workloads.make_workload(5)
    Bd, Hq, dd = dp.q.shape
    Hkv = dp.k_cache.shape[2]
    qd, kc, vc = (to_dev(x, "bf16", torch, dev) for x in (dp.q, dp.k_cache, dp.v_cache))
    sk = torch.from_numpy(dp.seqlens_k).to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((Bd, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_size(qd, kc, vc, chunk_keys=args.decode_chunk),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        fa.decode(qd, kc, vc, sk, scale=dp.scale, out=od, lse=lsed, workspace=ws,
                  chunk_keys=args.decode_chunk)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same prefill calls back to back, with no decode between them (outside
    # the timed steps; reported beside them, never as the value)
    n_b2b = max(5, args.steps // 2)
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev_b[0].record()
    for _ in range(n_b2b):
        fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse)
    ev_b[1].record()
    torch.cuda.synchronize()
    pre_b2b = ev_b[0].elapsed_time(ev_b[1]) / n_b2b

    # the ALiBi variants of both calls (slopes 2^(-8(h+1)/H)), timed the same way
    def alibi_slopes(H):
        return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32,
                            device=dev)
    sl_p, sl_d = alibi_slopes(H), alibi_slopes(Hq)
    n_alibi = max(3, args.steps // 4)
    fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse, alibi_slopes=sl_p)
    fa.decode(qd, kc, vc, sk, scale=dp.scale, out=od, lse=lsed, workspace=ws,
              chunk_keys=args.decode_chunk, alibi_slopes=sl_d)
    torch.cuda.synchronize()
    ev_a = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_alibi)]
    for e in ev_a:
        e[0].record()
        fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse, alibi_slopes=sl_p)
        e[1].record()
        fa.decode(qd, kc, vc, sk, scale=dp.scale, out=od, lse=lsed, workspace=ws,
                  chunk_keys=args.decode_chunk, alibi_slopes=sl_d)
        e[2].record()
    torch.cuda.synchronize()
    pre_a = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_a]))
    dec_a = float(np.mean([e[1].elapsed_time(e[2]) for e in ev_a]))

    # the prefill with RoPE (tables for base 10000 over all 128 dims): the
    # bf16 K rotation pass plus the attention kernel rotating Q at load
    half = d // 2
    inv = 10000.0 ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(N, dtype=np.float64)[:, None] * inv[None, :]
    rc = torch.from_numpy(np.cos(ang).astype(np.float32)).to(dev)
    rs = torch.from_numpy(np.sin(ang).astype(np.float32)).to(dev)
    wsr = torch.empty(fa.prefill_workspace_size(q, k, rope_cos=rc, rope_sin=rs), dtype=torch.uint8,
                      device=dev)
    fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse, rope_cos=rc, rope_sin=rs,
               workspace=wsr)
    torch.cuda.synchronize()
    ev_r = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_alibi)]
    for e in ev_r:
        e[0].record()
        fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse, rope_cos=rc, rope_sin=rs,
                   workspace=wsr)
        e[1].record()
    torch.cuda.synchronize()
    pre_r = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_r]))
    del wsr, rc, rs

    # the prefill with an explicit [1, 1, 1, N] additive mask (all zero: the
    # cost of reading a key-padding mask, the BERT page's layout)
    mzero = torch.zeros((1, 1, 1, N), dtype=torch.bfloat16, device=dev)
    fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse, attn_mask=mzero)
    torch.cuda.synchronize()
    ev_m = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_alibi)]
    for e in ev_m:
        e[0].record()
        fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse, attn_mask=mzero)
        e[1].record()
    torch.cuda.synchronize()
    pre_m = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_m]))

    # the same causal prefill in IEEE half (the FP16 of the BERT benchmark)
    ph = workloads.make_prefill(3, B, N, N, H, H, d, "f16", causal=True)
    qh, kh, vh = (torch.from_numpy(x.view(np.int16)).view(torch.float16).to(dev)
                  for x in (ph.q, ph.k, ph.v))
    oh = torch.empty_like(qh)
    fa.prefill(qh, kh, vh, causal=True, scale=ph.scale, out=oh, lse=lse)
    torch.cuda.synchronize()
    ev_h = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_alibi)]
    for e in ev_h:
        e[0].record()
        fa.prefill(qh, kh, vh, causal=True, scale=ph.scale, out=oh, lse=lse)
        e[1].record()
    torch.cuda.synchronize()
    pre_h = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_h]))
    del qh, kh, vh, oh

    # the decode over a paged pool holding the same logical cache
    page = 16
    pp = workloads.make_workload_paged(5, page)
    assert np.array_equal(pp.seqlens_k, dp.seqlens_k)
    qp, kp, vp = (to_dev(x, "bf16", torch, dev) for x in (pp.q, pp.k_pool, pp.v_pool))
    tab = torch.from_numpy(pp.block_table).to(dev)
    fa.decode(qp, kp, vp, sk, scale=pp.scale, out=od, lse=lsed, workspace=ws,
              chunk_keys=args.decode_chunk, block_table=tab)
    torch.cuda.synchronize()
    ev_p = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_alibi)]
    for e in ev_p:
        e[0].record()
        fa.decode(qp, kp, vp, sk, scale=pp.scale, out=od, lse=lsed, workspace=ws,
                  chunk_keys=args.decode_chunk, block_table=tab)
        e[1].record()
    torch.cuda.synchronize()
    dec_p = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_p]))
    table_bytes = 4 * int(sum(-(-int(L) // page) for L in pp.seqlens_k))
    del qp, kp, vp, tab

    # the decode over an FP8 E4M3 cache of the same draws (per-KV-head scales)
    fp = workloads.make_workload_fp8(5)
    assert np.array_equal(fp.seqlens_k, dp.seqlens_k)
    k8 = torch.from_numpy(fp.k_cache).to(dev).view(torch.float8_e4m3fn)
    v8 = torch.from_numpy(fp.v_cache).to(dev).view(torch.float8_e4m3fn)
    ks8 = torch.from_numpy(fp.k_scale).to(dev)
    vs8 = torch.from_numpy(fp.v_scale).to(dev)
    ws8 = torch.empty(fa.decode_workspace_size(qd, k8, v8, chunk_keys=args.decode_chunk,
                                               k_scale=ks8, v_scale=vs8), dtype=torch.uint8,
                      device=dev)
    fa.decode(qd, k8, v8, sk, scale=dp.scale, out=od, lse=lsed, workspace=ws8,
              chunk_keys=args.decode_chunk, k_scale=ks8, v_scale=vs8)
    torch.cuda.synchronize()
    ev_f = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_alibi)]
    for e in ev_f:
        e[0].record()
        fa.decode(qd, k8, v8, sk, scale=dp.scale, out=od, lse=lsed, workspace=ws8,
                  chunk_keys=args.decode_chunk, k_scale=ks8, v_scale=vs8)
        e[1].record()
    torch.cuda.synchronize()
    dec_f = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_f]))
    fp8_bytes = decode_bytes(dp.seqlens_k, Hq, Hkv, dd, kv_elt=1) + 2 * 4 * Hkv
    del k8, v8

    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    flops = prefill_flops(B, H, N, d)
    tflops = flops / (pre_ms.mean() * 1e-3) / 1e12
    dbytes = decode_bytes(dp.seqlens_k, Hq, Hkv, dd)
    gbs = dbytes / (dec_ms.mean() * 1e-3) / 1e9

    result = {
        "metric": "attention fwd TFLOP/s (causal N=8192,d=128) + decode HBM GB/s, % of roofline",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill B1 H32 N8192 d128 bf16 + decode B64 Hq32 Hkv8 d128 "
                        "bf16 KV lengths U[512,8192]",
            "prefill": {"batch": B, "heads": H, "seq_len": N, "head_dim": d, "causal": True},
            "decode": {"batch": Bd, "heads_q": Hq, "heads_kv": Hkv, "head_dim": dd,
                       "capacity": int(dp.k_cache.shape[1]),
                       "sum_kv_len": int(np.sum(dp.seqlens_k))},
            "parallelism": "single GPU",
        },
        "prefill": {"ms_mean": round(float(pre_ms.mean()), 4),
                    "ms_median": round(float(np.median(pre_ms)), 4),
                    "ms_min": round(float(pre_ms.min()), 4),
                    "algorithmic_flop": flops},
        "prefill_back_to_back": {"ms_mean": round(pre_b2b, 4),
                                 "tflops": round(flops / (pre_b2b * 1e-3) / 1e12, 2),
                                 "frac_of_bf16_peak": round(flops / (pre_b2b * 1e-3) / 1e12
                                                            / PEAK_BF16_TFLOPS, 4),
                                 "calls": n_b2b,
                                 "note": "the same prefill calls with no decode between them"},
        "decode": {"value": round(gbs, 1), "unit": "GB/s",
                   "ms_mean": round(float(dec_ms.mean()), 4),
                   "ms_median": round(float(np.median(dec_ms)), 4),
                   "ms_min": round(float(dec_ms.min()), 4),
                   "algorithmic_bytes": dbytes},
        "alibi": {"prefill_ms_mean": round(pre_a, 4),
                  "prefill_tflops": round(flops / (pre_a * 1e-3) / 1e12, 2),
                  "decode_ms_mean": round(dec_a, 4),
                  "decode_gbs": round(dbytes / (dec_a * 1e-3) / 1e9, 1),
                  "calls": n_alibi},
        "rope": {"rotary_dim": d, "prefill_ms_mean": round(pre_r, 4),
                 "prefill_tflops": round(flops / (pre_r * 1e-3) / 1e12, 2),
                 "note": "K rotation pass + attention with Q rotated at load", "calls": n_alibi},
        "f16": {"prefill_ms_mean": round(pre_h, 4),
                "prefill_tflops": round(flops / (pre_h * 1e-3) / 1e12, 2),
                "frac_of_f16_peak": round(flops / (pre_h * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "calls": n_alibi},
        "attn_mask": {"shape": [1, 1, 1, N], "prefill_ms_mean": round(pre_m, 4),
                      "prefill_tflops": round(flops / (pre_m * 1e-3) / 1e12, 2), "calls": n_alibi},
        "fp8_kv": {"format": "e4m3", "decode_ms_mean": round(dec_f, 4),
                   "decode_gbs": round(fp8_bytes / (dec_f * 1e-3) / 1e9, 1),
                   "frac_of_hbm_peak": round(fp8_bytes / (dec_f * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "speedup_vs_bf16_cache": round(float(dec_ms.mean()) / dec_f, 3),
                   "algorithmic_bytes": fp8_bytes, "calls": n_alibi},
        "paged": {"page_size": page, "num_pages": int(pp.k_pool.shape[0]),
                  "decode_ms_mean": round(dec_p, 4),
                  "decode_gbs": round((dbytes + table_bytes) / (dec_p * 1e-3) / 1e9, 1),
                  "calls": n_alibi},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(["prefill_bf16_kernel<128>"])},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "traffic": measured_traffic(["decode_split_kernel",
                                                         "decode_combine_kernel<128>"])},
        "host": platform.node(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p, args.cpu_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
