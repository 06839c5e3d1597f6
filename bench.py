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
library), so the per-call figures are kernel time plus launch gaps.

Outside the timed steps, each of the five workloads gets its own entry under
"configs": the tiny fp32 case, the BERT-shaped varlen encoder and the GQA
window prefill are timed on their own (warm-up calls, then one event pair per
call), and the two step workloads reuse the step's per-call events.  These
measurements, the variants below and the step's prefill called back to back
run first; the warm-up and timed steps run after them, so the steps start
on a GPU that has been busy rather than one ramping up from idle after input
generation (its first milliseconds of work otherwise run measurably slower).  Each
entry carries its throughput, its roofline fraction and the fp64 oracle timed
on the host's cores on the same inputs (the whole workload, or a stated
sample of its heads).  Further variants of the two step calls are timed the
same way: ALiBi ("alibi"), a paged pool of 16-row pages in shuffled order
("paged"), an FP8 E4M3 cache with per-KV-head scales ("fp8_kv"), RoPE over
all 128 dims ("rope"), an explicit [1, 1, 1, N] additive mask ("attn_mask")
and IEEE half ("f16", same draws rounded to half; the fp16 dense MFMA peak
equals bf16's).

Printed: ONE JSON line.  ``value`` is prefill throughput in TFLOP/s on the
algorithmic flop count (only visible (query, key) pairs: 4*d*H*N(N+1)/2);
decode throughput is reported beside it in GB/s on algorithmic bytes (each
valid K and V row read once per GQA group, plus Q, O, LSE, lengths).

``--summarize-profiles DIR`` turns the rocprofv3 CSV output of the profiling
runs named in ``profiles/*.md`` (subdirectories kt, fetch, write, clk of DIR)
into those summaries and ``profiles/traffic.json``; it needs no GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 (and fp16) MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector (256 CU x 2.4 GHz x 256 flop/clk)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


# ---------------------------------------------------------------------------
# algorithmic work of each workload
# ---------------------------------------------------------------------------
def prefill_flops(B, H, N, d):
    """Causal, Nq = Nk = N: 4 d flops per visible (query, key) pair."""
    return 4.0 * d * H * B * N * (N + 1) / 2.0


def pairs_visible(N, causal, window, seqlens_k=None, B=1):
    """Visible (query, key) pairs of one head, summed over the batch, for
    Nq = Nk = N with key lengths only (all query rows computed)."""
    total = 0
    for b in range(B):
        Lk = N if seqlens_k is None else int(seqlens_k[b])
        i = np.arange(N, dtype=np.int64)
        hi = np.minimum(Lk, i + 1) if causal else np.full(N, Lk)
        lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros(N, np.int64)
        total += int(np.maximum(hi - lo, 0).sum())
    return total


def prefill_bytes(B, Nq, Hq, d, elt, kv_rows, Hkv):
    """Q read, O written, LSE written, K and V rows read once."""
    return (2.0 * B * Nq * Hq * d * elt + 2.0 * kv_rows * Hkv * d * elt + 4.0 * B * Hq * Nq)


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timings (used for profiler runs)")
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="heads of the causal N=8192 workload the CPU oracle times")
    ap.add_argument("--decode-chunk", type=int, default=0,
                    help="keys per decode split (0 = library choice)")
    ap.add_argument("--no-clock-sample", action="store_true",
                    help="do not read the shader clock with amd-smi during the run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/*.md and profiles/traffic.json from rocprofv3 CSVs "
                         "under DIR (no GPU needed) and exit")
    return ap.parse_args()


def to_dev(a, dtype, torch, dev):
    if dtype in ("bf16", "f16"):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


# ---------------------------------------------------------------------------
# CPU oracle baselines
# ---------------------------------------------------------------------------
def host_info():
    info = {"cores": len(os.sched_getaffinity(0)), "cpu": "unknown", "blas": "unknown",
            "blas_threads": None}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                info["blas"] = f"{i.get('internal_api')} {i.get('version')}"
                info["blas_threads"] = int(i.get("num_threads", 1))
                break
    except Exception:  # pragma: no cover
        pass
    return info


def cpu_time(fn, repeats):
    """Median wall seconds of ``repeats`` runs (one run when it is long)."""
    times = []
    for r in range(repeats):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if r == 0 and times[0] > 8.0:
            break
    return float(np.median(times)), len(times)


def cpu_entry(value, unit, seconds, runs, sample, info):
    return {"value": value, "unit": unit, "cores": info["blas_threads"] or info["cores"],
            "kind": "oracle", "seconds": round(seconds, 4), "runs": runs,
            "sample": f"{sample}; fp64 NumPy three-step oracle, median of {runs} run(s), "
                      f"{info['cpu']}, BLAS {info['blas']} with {info['blas_threads']} threads, "
                      f"affinity {info['cores']} cpus"}


def cpu_prefill(p, flops_per_head_pair, heads, batches, sample, info, repeats):
    """Time the oracle on the given (batch, head) sample of a prefill workload;
    ``flops_per_head_pair[b]`` is the algorithmic flop count of one head of
    sequence b."""
    import oracle
    import workloads
    sub = [(b, tuple(heads)) for b in batches]
    data = [(workloads.to_f64(p.q[b:b + 1], p.dtype), workloads.to_f64(p.k[b:b + 1], p.dtype),
             workloads.to_f64(p.v[b:b + 1], p.dtype)) for b, _ in sub]

    def run():
        for (b, hs), (q, k, v) in zip(sub, data):
            oracle.attention(q, k, v, scale=p.scale, causal=p.causal, window_left=p.window_left,
                             seqlens_q=None if p.seqlens_q is None else p.seqlens_q[b:b + 1],
                             seqlens_k=None if p.seqlens_k is None else p.seqlens_k[b:b + 1],
                             heads=list(hs))
    sec, runs = cpu_time(run, repeats)
    flops = sum(flops_per_head_pair[b] * len(hs) for b, hs in sub)
    return cpu_entry(flops / sec / 1e12, "TFLOP/s", sec, runs, sample, info)


def cpu_decode(dp, nbytes, info, repeats):
    import oracle
    import workloads
    q = workloads.to_f64(dp.q, dp.dtype)
    kc = workloads.bf16_bits_to_f32(dp.k_cache)
    vc = workloads.bf16_bits_to_f32(dp.v_cache)
    sec, runs = cpu_time(lambda: oracle.decode(q, kc, vc, dp.seqlens_k, scale=dp.scale), repeats)
    return cpu_entry(nbytes / sec / 1e9, "GB/s", sec, runs,
                     f"the whole workload ({len(dp.seqlens_k)} sequences)", info)


# ---------------------------------------------------------------------------
# GPU timing helpers
# ---------------------------------------------------------------------------
def warm_up(torch, fns, warm, warm_ms):
    """Untimed calls: at least ``warm`` rounds of ``fns`` and at least
    ``warm_ms`` of wall time with the GPU kept busy.  After the host has left
    the GPU idle (input generation), its clock takes milliseconds to come
    back up; a fixed count of a short call ends before that."""
    t0 = time.perf_counter()
    k = 0
    while k < warm or (time.perf_counter() - t0) * 1e3 < warm_ms:
        for f in fns:
            f()
        k += 1
        if k % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_calls(torch, fn, n, warm=3, warm_ms=25.0):
    """Per-call HIP-event times (ms) of ``fn`` on the current stream."""
    warm_up(torch, [fn], warm, warm_ms)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for e in ev:
        e[0].record()
        fn()
        e[1].record()
    torch.cuda.synchronize()
    return np.array([e[0].elapsed_time(e[1]) for e in ev])


def time_pairs(torch, fa_, fb_, n, warm=3, warm_ms=25.0):
    """Per-call HIP-event times (ms) of ``fa_`` and ``fb_`` called alternately
    (a, b, a, b, ...), so that both see the same clock and the same preceding
    work."""
    warm_up(torch, [fa_, fb_], warm, warm_ms)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    for e in ev:
        e[0].record()
        fa_()
        e[1].record()
        e[2].record()
        fb_()
        e[3].record()
    torch.cuda.synchronize()
    return (np.array([e[0].elapsed_time(e[1]) for e in ev]),
            np.array([e[2].elapsed_time(e[3]) for e in ev]))


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def start_clock_sampler(seconds):
    """Start a child process group that reads the shader clocks (one value per
    XCD) with a single amd-smi call about every second.  Started before this
    process makes its first GPU call; skipped under a profiler (its injected
    library would follow the child) or when amd-smi is missing.  Returns a
    handle or None."""
    import shutil
    import subprocess
    import tempfile
    if any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ) or \
            "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe) or not shutil.which("bash"):
        return None
    out = tempfile.NamedTemporaryFile(prefix="fa_bench_sclk_", suffix=".json", delete=False)
    # the loop ends on its own once this process is gone or after `seconds`
    loop = (f"while kill -0 {os.getpid()} 2>/dev/null && [ $SECONDS -lt {int(seconds)} ]; do "
            f"echo \"@T $(date +%s.%N)\"; '{exe}' metric -g 0 --clock --json; sleep 0.5; done")
    try:
        proc = subprocess.Popen(["bash", "-c", loop], stdout=out, stderr=subprocess.DEVNULL,
                                stdin=subprocess.DEVNULL, start_new_session=True)
    except OSError:
        out.close()
        os.unlink(out.name)
        return None
    import atexit
    atexit.register(_stop_group, proc)
    return proc, out


def _stop_group(proc):
    import signal
    if proc.poll() is None:
        try:
            os.killpg(proc.pid, signal.SIGTERM)      # the loop and its current amd-smi call
        except OSError:
            pass


def finish_clock_sampler(handle, windows=None):
    """Stop the sampler and summarise the shader clocks it read while the GPU
    was busy (samples of 1000 MHz or more; an idle GPU reads about 100), over
    the whole run and inside each named (start, end) time window."""
    if handle is None:
        return None
    proc, out = handle
    _stop_group(proc)
    try:
        proc.wait(timeout=10)
    except Exception:
        proc.kill()
        proc.wait()
    out.close()
    try:
        with open(out.name) as f:
            text = f.read()
    finally:
        os.unlink(out.name)
    # each amd-smi call follows a "@T <unix time>" line written just before it
    samples = []                                    # (time, MHz)
    for part in re.split(r"^@T ", text, flags=re.M)[1:]:
        head, _, body = part.partition("\n")
        try:
            t = float(head.strip())
        except ValueError:
            continue
        for v in re.findall(r'"gfx_\d+":\s*\{\s*"clk":\s*\{\s*"value":\s*(\d+)', body):
            samples.append((t, int(v)))

    def stats(vals):
        busy = sorted(v for v in vals if v >= 1000)
        d = {"samples": len(vals), "busy_samples": len(busy)}
        if busy:
            d.update({"busy_median_mhz": busy[len(busy) // 2], "busy_min_mhz": busy[0],
                      "busy_max_mhz": busy[-1]})
        return d

    summary = {"tool": "amd-smi metric --clock about twice a second, every XCD"}
    summary.update(stats([v for _, v in samples]))
    for name, (t0, t1) in (windows or {}).items():
        summary[name] = stats([v for t, v in samples if t0 <= t <= t1])
    return summary


def ms_stats(ms):
    return {"ms_mean": round(float(ms.mean()), 4), "ms_median": round(float(np.median(ms)), 4),
            "ms_min": round(float(ms.min()), 4), "calls": int(len(ms))}


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    sampler = None if (args.copy_calibration or args.no_clock_sample) else start_clock_sampler(900)

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

    # ---- inputs of the step (seeded, generated once, resident in HBM) -------
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

    n_var = 20                                  # calls per variant timing
    # the step's prefill called back to back, with no decode between the calls
    # (reported beside the steps, never as the value); measured first, so the
    # later measurements start on a GPU that is already busy.  The GPU idled
    # while the host drew the inputs, and its clock takes some milliseconds to
    # come back up: 30 untimed calls (at least 25 ms) go first, and every
    # per-call timing below starts with at least 25 ms of untimed calls.
    n_b2b = 50
    pre_bb = time_calls(torch, lambda: fa.prefill(q, k, v, causal=True, scale=p.scale, out=o,
                                                   lse=lse), n_b2b, warm=30)
    pre_b2b = float(np.mean(pre_bb))
    # ---- the other three workloads, each timed on its own -------------------
    # tiny fp32 single head, B1 H1 N128 d64, non-causal
    p1 = workloads.make_workload(1)
    q1, k1, v1 = (to_dev(x, "f32", torch, dev) for x in (p1.q, p1.k, p1.v))
    o1 = torch.empty_like(q1)
    l1 = torch.empty((1, 1, 128), dtype=torch.float32, device=dev)
    ms1 = time_calls(torch, lambda: fa.prefill(q1, k1, v1, scale=p1.scale, out=o1, lse=l1), 50)
    N1, d1 = p1.q.shape[1], p1.q.shape[3]
    fl1 = 4.0 * d1 * N1 * N1
    by1 = prefill_bytes(1, N1, 1, d1, 4, N1, 1)

    # BERT-shaped B8 H12 N512 d64 bf16, key lengths U[128, 512], all query rows
    p2 = workloads.make_workload(2)
    B2, N2, H2, d2 = p2.q.shape
    q2, k2, v2 = (to_dev(x, "bf16", torch, dev) for x in (p2.q, p2.k, p2.v))
    sk2 = torch.from_numpy(p2.seqlens_k).to(dev)
    o2 = torch.empty_like(q2)
    l2 = torch.empty((B2, H2, N2), dtype=torch.float32, device=dev)
    ms2 = time_calls(torch, lambda: fa.prefill(q2, k2, v2, scale=p2.scale, seqlens_k=sk2, out=o2,
                                               lse=l2), 50)
    pairs2 = [pairs_visible(N2, False, -1, p2.seqlens_k[b:b + 1]) for b in range(B2)]
    fl2 = 4.0 * d2 * H2 * sum(pairs2)
    by2 = prefill_bytes(B2, N2, H2, d2, 2, int(np.sum(p2.seqlens_k)), H2) + 4 * B2

    # GQA causal window 1024, B2 Hq32 Hkv8 N4096 d128 bf16
    p4 = workloads.make_workload(4)
    B4, N4, H4, d4 = p4.q.shape
    Hkv4 = p4.k.shape[2]
    q4, k4, v4 = (to_dev(x, "bf16", torch, dev) for x in (p4.q, p4.k, p4.v))
    o4 = torch.empty_like(q4)
    l4 = torch.empty((B4, H4, N4), dtype=torch.float32, device=dev)
    ms4 = time_calls(torch, lambda: fa.prefill(q4, k4, v4, causal=True, window=p4.window_left,
                                               scale=p4.scale, out=o4, lse=l4), 30)
    pairs4 = pairs_visible(N4, True, p4.window_left)
    fl4 = 4.0 * d4 * H4 * B4 * pairs4
    by4 = prefill_bytes(B4, N4, H4, d4, 2, B4 * N4, Hkv4)
    del q1, k1, v1, o1, q2, k2, v2, o2, q4, k4, v4, o4

    # ---- variants of the step's two calls ------------------------------------
    def alibi_slopes(H):
        return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32,
                            device=dev)
    sl_p, sl_d = alibi_slopes(H), alibi_slopes(Hq)
    pre_a = time_calls(torch, lambda: fa.prefill(q, k, v, causal=True, scale=p.scale, out=o,
                                                 lse=lse, alibi_slopes=sl_p), n_var, 1)
    dec_a = time_calls(torch, lambda: fa.decode(qd, kc, vc, sk, scale=dp.scale, out=od, lse=lsed,
                                                workspace=ws, chunk_keys=args.decode_chunk,
                                                alibi_slopes=sl_d), n_var, 1)

    # RoPE (tables for base 10000 over all 128 dims)
    half = d // 2
    inv = 10000.0 ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(N, dtype=np.float64)[:, None] * inv[None, :]
    rc = torch.from_numpy(np.cos(ang).astype(np.float32)).to(dev)
    rs = torch.from_numpy(np.sin(ang).astype(np.float32)).to(dev)
    wsr = torch.empty(max(16, fa.prefill_workspace_size(q, k, rope_cos=rc, rope_sin=rs)),
                      dtype=torch.uint8, device=dev)
    # timed alternately with the plain call, so that the ratio does not depend
    # on what ran before (the ALiBi decode just before lowers the clock)
    pre_rp, pre_r = time_pairs(torch, lambda: fa.prefill(q, k, v, causal=True, scale=p.scale, out=o,
                                                         lse=lse),
                               lambda: fa.prefill(q, k, v, causal=True, scale=p.scale, out=o,
                                                  lse=lse, rope_cos=rc, rope_sin=rs,
                                                  workspace=wsr), n_var)
    del wsr, rc, rs

    # an explicit [1, 1, 1, N] additive mask (all zero: the cost of reading a
    # key-padding mask, the BERT page's layout)
    mzero = torch.zeros((1, 1, 1, N), dtype=torch.bfloat16, device=dev)
    pre_m = time_calls(torch, lambda: fa.prefill(q, k, v, causal=True, scale=p.scale, out=o,
                                                 lse=lse, attn_mask=mzero), n_var, 1)

    # the same causal prefill in IEEE half (the FP16 of the BERT benchmark)
    ph = workloads.make_prefill(3, B, N, N, H, H, d, "f16", causal=True)
    qh, kh, vh = (to_dev(x, "f16", torch, dev) for x in (ph.q, ph.k, ph.v))
    oh = torch.empty_like(qh)
    pre_h = time_calls(torch, lambda: fa.prefill(qh, kh, vh, causal=True, scale=ph.scale, out=oh,
                                                 lse=lse), n_var, 1)
    del qh, kh, vh, oh

    # the decode over a paged pool holding the same logical cache
    page = 16
    pp = workloads.make_workload_paged(5, page)
    assert np.array_equal(pp.seqlens_k, dp.seqlens_k)
    qp, kp, vp = (to_dev(x, "bf16", torch, dev) for x in (pp.q, pp.k_pool, pp.v_pool))
    tab = torch.from_numpy(pp.block_table).to(dev)
    dec_p = time_calls(torch, lambda: fa.decode(qp, kp, vp, sk, scale=pp.scale, out=od, lse=lsed,
                                                workspace=ws, chunk_keys=args.decode_chunk,
                                                block_table=tab), n_var, 1)
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
    dec_f = time_calls(torch, lambda: fa.decode(qd, k8, v8, sk, scale=dp.scale, out=od, lse=lsed,
                                                workspace=ws8, chunk_keys=args.decode_chunk,
                                                k_scale=ks8, v_scale=vs8), n_var, 1)
    fp8_bytes = decode_bytes(dp.seqlens_k, Hq, Hkv, dd, kv_elt=1) + 2 * 4 * Hkv
    del k8, v8

    # ---- the timed steps: last, on a GPU the measurements above kept busy --
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
    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in events])

    # ---- figures ---------------------------------------------------------------
    flops = prefill_flops(B, H, N, d)
    tflops = flops / (pre_ms.mean() * 1e-3) / 1e12
    dbytes = decode_bytes(dp.seqlens_k, Hq, Hkv, dd)
    gbs = dbytes / (dec_ms.mean() * 1e-3) / 1e9
    by3 = prefill_bytes(B, N, H, d, 2, B * N, H)

    def tf(fl, ms):
        return fl / (ms * 1e-3) / 1e12

    configs = {
        "config1": {"workload": "B1 H1 N128 d64 fp32, not causal", **ms_stats(ms1),
                    "algorithmic_flop": fl1, "algorithmic_bytes": by1,
                    "tflops": round(tf(fl1, ms1.mean()), 4),
                    "roofline": roofline("alu", tf(fl1, ms1.mean()), PEAK_F32_TFLOPS, "TFLOP/s",
                                         measured_traffic(["prefill_f32_kernel<64>"])),
                    "note": "4 lanes per query row, 16 rows per workgroup (8 workgroups): "
                            "latency-bound; fp32 vector peak"},
        "config2": {"workload": "B8 H12 N512 d64 bf16, key lengths U[128,512] "
                                f"(sum {int(np.sum(p2.seqlens_k))}), all query rows",
                    **ms_stats(ms2), "algorithmic_flop": fl2, "algorithmic_bytes": by2,
                    "tflops": round(tf(fl2, ms2.mean()), 2),
                    "roofline": roofline("mfma", tf(fl2, ms2.mean()), PEAK_BF16_TFLOPS, "TFLOP/s",
                                         measured_traffic([K_PREFILL_D64])),
                    "roofline_hbm": roofline("hbm", by2 / (ms2.mean() * 1e-3) / 1e9, PEAK_HBM_GBS,
                                             "GB/s")},
        "config3": {"workload": "B1 H32 N8192 d128 bf16 causal (the step's prefill)",
                    **ms_stats(pre_ms), "algorithmic_flop": flops, "algorithmic_bytes": by3,
                    "tflops": round(tflops, 2),
                    "roofline": roofline("mfma", tflops, PEAK_BF16_TFLOPS, "TFLOP/s",
                                         measured_traffic([K_PREFILL]))},
        "config4": {"workload": "B2 Hq32 Hkv8 N4096 d128 bf16 causal, window 1024",
                    **ms_stats(ms4), "algorithmic_flop": fl4, "algorithmic_bytes": by4,
                    "tflops": round(tf(fl4, ms4.mean()), 2),
                    "roofline": roofline("mfma", tf(fl4, ms4.mean()), PEAK_BF16_TFLOPS, "TFLOP/s",
                                         measured_traffic([K_PREFILL_GQA]))},
        "config5": {"workload": "decode B64 Hq32 Hkv8 d128 bf16, KV lengths U[512,8192] "
                                f"(sum {int(np.sum(dp.seqlens_k))}) (the step's decode)",
                    **ms_stats(dec_ms), "algorithmic_bytes": dbytes, "gbs": round(gbs, 1),
                    "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                         measured_traffic([K_DECODE, K_COMBINE]))},
    }

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
        "prefill": {**ms_stats(pre_ms), "algorithmic_flop": flops},
        "prefill_back_to_back": {"ms_mean": round(pre_b2b, 4),
                                 "ms_median": round(float(np.median(pre_bb)), 4),
                                 "tflops": round(flops / (pre_b2b * 1e-3) / 1e12, 2),
                                 "frac_of_bf16_peak": round(flops / (pre_b2b * 1e-3) / 1e12
                                                            / PEAK_BF16_TFLOPS, 4),
                                 "calls": n_b2b,
                                 "note": "the same prefill calls with no decode between them"},
        "decode": {"value": round(gbs, 1), "unit": "GB/s", **ms_stats(dec_ms),
                   "algorithmic_bytes": dbytes},
        "configs": configs,
        "alibi": {"prefill_ms_mean": round(float(pre_a.mean()), 4),
                  "prefill_tflops": round(tf(flops, pre_a.mean()), 2),
                  "decode_ms_mean": round(float(dec_a.mean()), 4),
                  "decode_gbs": round(dbytes / (dec_a.mean() * 1e-3) / 1e9, 1), "calls": n_var},
        "rope": {"rotary_dim": d, "prefill_ms_mean": round(float(pre_r.mean()), 4),
                 "prefill_tflops": round(tf(flops, pre_r.mean()), 2),
                 "plain_interleaved_ms_mean": round(float(pre_rp.mean()), 4),
                 "vs_plain_interleaved": round(float(pre_r.mean() / pre_rp.mean()), 4),
                 "note": "K rotation pass + attention with Q rotated at load; timed alternately "
                         "with the plain call",
                 "calls": n_var},
        "f16": {"prefill_ms_mean": round(float(pre_h.mean()), 4),
                "prefill_tflops": round(tf(flops, pre_h.mean()), 2),
                "frac_of_f16_peak": round(tf(flops, pre_h.mean()) / PEAK_BF16_TFLOPS, 4),
                "calls": n_var},
        "attn_mask": {"shape": [1, 1, 1, N], "prefill_ms_mean": round(float(pre_m.mean()), 4),
                      "prefill_tflops": round(tf(flops, pre_m.mean()), 2), "calls": n_var},
        "fp8_kv": {"format": "e4m3", "decode_ms_mean": round(float(dec_f.mean()), 4),
                   "decode_gbs": round(fp8_bytes / (dec_f.mean() * 1e-3) / 1e9, 1),
                   "frac_of_hbm_peak": round(fp8_bytes / (dec_f.mean() * 1e-3) / 1e9
                                             / PEAK_HBM_GBS, 4),
                   "speedup_vs_bf16_cache": round(float(dec_ms.mean() / dec_f.mean()), 3),
                   "algorithmic_bytes": fp8_bytes, "calls": n_var,
                   "traffic": measured_traffic([K_DECODE_FP8, K_COMBINE])},
        "paged": {"page_size": page, "num_pages": int(pp.k_pool.shape[0]),
                  "decode_ms_mean": round(float(dec_p.mean()), 4),
                  "decode_gbs": round((dbytes + table_bytes) / (dec_p.mean() * 1e-3) / 1e9, 1),
                  "calls": n_var},
        "roofline": configs["config3"]["roofline"],
        "roofline_decode": configs["config5"]["roofline"],
        "host": platform.node(),
    }
    # shader clock over the GPU part of the run, and inside a window of about
    # 4 s of back-to-back calls of the causal N = 8192 prefill (none under a
    # profiler)
    windows = {}
    if sampler is not None:
        n_calls = max(1, int(4000.0 / max(float(pre_ms.mean()), 1e-3)))
        t_start = time.time()
        for _ in range(n_calls):
            fa.prefill(q, k, v, causal=True, scale=p.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        # an amd-smi call reads the clock a few tenths of a second after its timestamp
        windows["prefill_window"] = (t_start + 0.2, time.time() - 1.0)
    result["sclk"] = finish_clock_sampler(sampler, windows)

    if not args.no_cpu_baseline:
        info = host_info()
        # the oracle on each workload, after all GPU timing
        fl_head1 = [4.0 * d1 * N1 * N1]
        configs["config1"]["cpu_baseline"] = cpu_prefill(
            p1, fl_head1, range(1), [0], "the whole workload", info, 3)
        fl_head2 = [4.0 * d2 * x for x in pairs2]
        configs["config2"]["cpu_baseline"] = cpu_prefill(
            p2, fl_head2, range(H2), range(B2), "the whole workload (8 sequences x 12 heads)",
            info, 3)
        fl_head3 = [4.0 * d * N * (N + 1) / 2.0]
        hs = range(args.cpu_heads)
        configs["config3"]["cpu_baseline"] = cpu_prefill(
            p, fl_head3, hs, [0], f"heads 0-{args.cpu_heads - 1} of 32 (all 8192 rows each)",
            info, 1)
        fl_head4 = [4.0 * d4 * pairs4] * B4
        configs["config4"]["cpu_baseline"] = cpu_prefill(
            p4, fl_head4, range(8), [0], "sequence 0, heads 0-7 of 32 (all 4096 rows each)",
            info, 1)
        configs["config5"]["cpu_baseline"] = cpu_decode(dp, dbytes, info, 3)
        result["cpu_baseline"] = configs["config3"]["cpu_baseline"]
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# profile summaries (no GPU): rocprofv3 CSV -> profiles/*.md, traffic.json
# ---------------------------------------------------------------------------
PROFILE_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 {opts} -d <out>/{sub} "
               "--output-format csv -- python3 /root/repo/bench.py --steps 3 --warmup 1 "
               "--no-cpu-baseline")
# kernels (exact template names of the kernel trace) whose counter-measured
# HBM bytes the JSON line reports
K_PREFILL = "prefill_bf16_kernel<128, false, false, 0, false, false, false>"
K_PREFILL_GQA = "prefill_bf16_kernel<128, false, false, 0, false, true, true>"
K_PREFILL_D64 = "prefill_bf16_kernel<64, false, false, 0, false, false, false>"
K_DECODE = "decode_split_kernel<128, 4, false, false, false, 16, false>"
K_DECODE_FP8 = "decode_split_fp8_kernel<128, 4, false, false, 32, false>"
K_COMBINE = "decode_combine_kernel<128, false>"
CTR1 = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA",
        "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_MFMA_MOPS_BF16"]
CTR2 = ["SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY",
        "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"]
CALIB_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc {c} -d <out>/{sub} "
             "--output-format csv -- python3 /root/repo/bench.py --copy-calibration")
# copy calibration: counter KiB per 1 GiB read (FETCH) or written (WRITE),
# re-read from the calibration runs when they are present
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0
CSRC = "transformer_attention_flashattention_amd/csrc/"


def _short(n):
    import re
    n = n.replace("void fa::(anonymous namespace)::", "")
    return re.sub(r"\(fa::\w+\)$", "", n)


def _one(pattern):
    import glob
    f = glob.glob(pattern)
    if len(f) != 1:
        raise SystemExit(f"expected one file for {pattern}, found {f}")
    return f[0]


def _counter_means(path, cname):
    import collections
    import csv
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == cname:
            acc[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: float(np.mean(v)) for k, v in acc.items()}


def summarize_profiles(out):
    """Summaries of one profiling session: <out>/kt (kernel trace), <out>/fetch
    and <out>/write (HBM counters), <out>/clk (clock counters), and optionally
    <out>/calib_fetch, <out>/calib_write (a plain 1 GiB copy)."""
    import collections
    import csv
    import glob
    import hashlib
    prof = os.path.join(ROOT, "profiles")
    wl = ("bench workload (causal prefill B1 H32 N8192 d128 bf16 + decode B64 Hq32 Hkv8 "
          "d128 bf16, then the other workloads and variants bench.py times)")

    # kernel trace
    rows = list(csv.DictReader(open(_one(f"{out}/kt/*/*_kernel_stats.csv"))))
    # per-dispatch durations (for the median: the average also holds the
    # first calls after the GPU idled, whose clock is still rising)
    durs = collections.defaultdict(list)
    for r in csv.DictReader(open(_one(f"{out}/kt/*/*_kernel_trace.csv"))):
        durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# Kernel trace: {wl}", "",
             "Command (one warm-up step and three timed steps of bench.py, then everything else "
             "it times):", "", "    " + PROFILE_CMD.format(opts="--kernel-trace --stats", sub="kt"),
             "", "Summarised by `python bench.py --summarize-profiles <out>` (the median from the "
             "per-dispatch trace).", "",
             "| kernel | calls | average us | median us | min us | max us | share |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        d = durs.get(r["Name"])
        med = f"{float(np.median(d)):.1f}" if d else "-"
        lines.append(f"| {_short(r['Name'])[:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} "
                     f"| {med} | {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} "
                     f"| {float(r['Percentage']):.1f}% |")
    open(os.path.join(prof, "bench_workload_kernel_trace.md"), "w").write("\n".join(lines) + "\n")

    # HBM traffic, scaled by the copy calibration
    ff, wf = FETCH_FACTOR, WRITE_FACTOR
    cal = ""
    cf = glob.glob(f"{out}/calib_fetch/*/*_counter_collection.csv")
    cw = glob.glob(f"{out}/calib_write/*/*_counter_collection.csv")
    if cf and cw:
        cfk = max(_counter_means(cf[0], "FETCH_SIZE").values())
        cwk = max(_counter_means(cw[0], "WRITE_SIZE").values())
        ff, wf = (1 << 20) / cfk, (1 << 20) / cwk
        cal = (f"FETCH_SIZE reads {cfk:.0f} KiB for 1048576 KiB read: factor {ff:.3f}; "
               f"WRITE_SIZE reads {cwk:.0f} KiB for 1048576 KiB written: factor {wf:.3f}.")
    fetch = _counter_means(_one(f"{out}/fetch/*/*_counter_collection.csv"), "FETCH_SIZE")
    write = _counter_means(_one(f"{out}/write/*/*_counter_collection.csv"), "WRITE_SIZE")
    lines = [f"# HBM traffic per launch: {wl}", "",
             "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the dispatches of "
             "each kernel), each from its own run:", "",
             "    " + PROFILE_CMD.format(opts="--pmc FETCH_SIZE", sub="fetch"),
             "    " + PROFILE_CMD.format(opts="--pmc WRITE_SIZE", sub="write"), "",
             "Calibration: a plain 1 GiB device copy (reads 1 GiB, writes 1 GiB), same counters:", "",
             "    " + CALIB_CMD.format(c="FETCH_SIZE", sub="calib_fetch"),
             "    " + CALIB_CMD.format(c="WRITE_SIZE", sub="calib_write"), "",
             cal or f"Factors {ff:.3f} (FETCH_SIZE) and {wf:.3f} (WRITE_SIZE) from an earlier "
                    "calibration run.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (scaled) | HBM write MB (scaled) |",
             "|---|---|---|---|---|"]
    for kname in fetch:
        if not kname.startswith(("prefill", "decode", "rope")):
            continue
        lines.append(f"| {kname[:70]} | {fetch[kname]:.0f} | {write.get(kname, 0):.0f} "
                     f"| {fetch[kname] * 1024 * ff / 1e6:.1f} | {write.get(kname, 0) * 1024 * wf / 1e6:.1f} |")
    open(os.path.join(prof, "bench_workload_hbm_traffic.md"), "w").write("\n".join(lines) + "\n")

    def sha(srcs):
        h = hashlib.sha256()
        for s in srcs:
            h.update(open(os.path.join(ROOT, s), "rb").read())
        return h.hexdigest()
    kern = {}

    def ent(key, name, srcs):
        kern[key] = {"name": name, "fetch_bytes": int(fetch[name] * 1024 * ff),
                     "write_bytes": int(write[name] * 1024 * wf),
                     "traffic_bytes": int(fetch[name] * 1024 * ff + write[name] * 1024 * wf),
                     "sources": srcs, "sources_sha256": sha(srcs)}
    pf = [CSRC + "prefill_bf16.hip", CSRC + "fa_internal.h"]
    dc = [CSRC + "decode_bf16.hip", CSRC + "fa_internal.h", CSRC + "fa_api.cpp"]
    for kname in fetch:
        if kname.startswith("prefill_bf16"):
            ent(kname, kname, pf)
        elif kname.startswith("prefill_f32"):
            ent(kname, kname, [CSRC + "prefill_f32.hip", CSRC + "fa_internal.h"])
        elif kname.startswith("decode"):
            ent(kname, kname, dc)
        elif kname.startswith("rope"):
            ent(kname, kname, [CSRC + "rope_bf16.hip", CSRC + "fa_internal.h"])
    json.dump({"calibration": {"fetch_factor": ff, "write_factor": wf, "copy_bytes": 1 << 30},
               "kernels": kern}, open(os.path.join(prof, "traffic.json"), "w"), indent=1)

    # shader clock per dispatch: GRBM_COUNT / 8 XCDs / duration
    clk = glob.glob(f"{out}/clk/*/*_counter_collection.csv")
    if clk:
        kt = {r["Dispatch_Id"]: r for r in csv.DictReader(open(_one(f"{out}/clk/*/*_kernel_trace.csv")))}
        acc = collections.defaultdict(dict)
        for r in csv.DictReader(open(clk[0])):
            acc[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
        per = collections.defaultdict(list)
        for did, c in acc.items():
            t = kt[did]
            dur = int(t["End_Timestamp"]) - int(t["Start_Timestamp"])
            per[_short(t["Kernel_Name"])].append((dur, c["GRBM_COUNT"]))
        lines = [f"# Shader clock under load: {wl}", "",
                 "GRBM_COUNT counts clock cycles of each of the 8 XCDs while a dispatch runs, so "
                 "GRBM_COUNT / 8 / duration is the average shader clock. Kernels shorter than "
                 "100 us are left out (there the count and the duration are too coarse).", "",
                 "    " + PROFILE_CMD.format(opts="--pmc GRBM_COUNT GRBM_GUI_ACTIVE --kernel-trace",
                                             sub="clk"), "",
                 "| kernel | dispatches | average us (under counters) | cycles per XCD (M) | clock GHz |",
                 "|---|---|---|---|---|"]
        for kname, vals in sorted(per.items(), key=lambda kv: -np.mean([x[0] for x in kv[1]])):
            dm = float(np.mean([x[0] for x in vals]))
            if dm < 100000:
                continue
            cyc = float(np.mean([x[1] for x in vals])) / 8
            ghz = float(np.median([x[1] / 8 / x[0] for x in vals]))
            lines.append(f"| {kname[:70]} | {len(vals)} | {dm / 1e3:.1f} | {cyc / 1e6:.3f} | {ghz:.3f} |")
        open(os.path.join(prof, "bench_workload_clock.md"), "w").write("\n".join(lines) + "\n")
    # shader counters: two runs (each within the per-block counter limits)
    c1 = glob.glob(f"{out}/ctr1/*/*_counter_collection.csv")
    c2 = glob.glob(f"{out}/ctr2/*/*_counter_collection.csv")
    if c1 and c2:
        vals = collections.defaultdict(lambda: collections.defaultdict(float))
        order = []
        for run, f in (("ctr1", c1[0]), ("ctr2", c2[0])):
            for r in csv.DictReader(open(f)):
                k = _short(r["Kernel_Name"])
                if not k.startswith(("prefill", "decode", "rope")):
                    continue
                if k not in order:
                    order.append(k)
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and run == "ctr2":
                    continue
                vals[k][(r["Counter_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
        lines = [f"# Shader counters: {wl}", "",
                 "Two runs (the counters of one run stay within the per-block limits):", "",
                 "    " + PROFILE_CMD.format(opts="--pmc " + " ".join(CTR1), sub="ctr1"),
                 "    " + PROFILE_CMD.format(opts="--pmc " + " ".join(CTR2), sub="ctr2"), "",
                 "Values are per dispatch (averaged over the dispatches of each kernel), summed over "
                 "the chip as the counters report them.  Ratios: VALU and LDS instructions per MFMA "
                 "instruction, and the share of wave cycles spent waiting (SQ_WAIT_ANY / "
                 "SQ_WAVE_CYCLES)."]
        for k in order:
            per = collections.defaultdict(list)
            for (c, _), v in vals[k].items():
                per[c].append(v)
            mean = {c: float(np.mean(v)) for c, v in per.items()}
            lines += ["", f"## {k}", "", "| counter | value |", "|---|---|"]
            lines += [f"| {c} | {mean[c]:.0f} |" for c in sorted(mean)]
            if mean.get("SQ_INSTS_MFMA"):
                lines.append(f"| VALU / MFMA | {mean.get('SQ_INSTS_VALU', 0) / mean['SQ_INSTS_MFMA']:.2f} |")
                lines.append(f"| LDS / MFMA | {mean.get('SQ_INSTS_LDS', 0) / mean['SQ_INSTS_MFMA']:.2f} |")
            if mean.get("SQ_WAVE_CYCLES"):
                lines.append(f"| wait share | {mean.get('SQ_WAIT_ANY', 0) / mean['SQ_WAVE_CYCLES']:.2f} |")
        open(os.path.join(prof, "bench_workload_counters.md"), "w").write("\n".join(lines) + "\n")
    print(open(os.path.join(prof, "bench_workload_kernel_trace.md")).read())


if __name__ == "__main__":
    main()
