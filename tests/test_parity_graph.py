"""GPU: the library's calls inside a captured HIP graph.  The entry points
allocate nothing and issue no memset, so a capture of a prefill and a decode
call replays correctly; every replay, with eager work and synchronisation in
between, must match the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import DEV, decode_inputs, prefill_inputs, say

pytestmark = pytest.mark.gpu


def test_prefill_and_decode_replay_in_a_graph():
    p = workloads.make_prefill(140, 2, 300, 300, 8, 2, 128, "bf16", causal=True,
                               seqlens_k_range=(100, 300), seqlens_q_equal_k=True)
    dp = workloads.make_decode(141, 4, 8, 2, 128, 900, (1, 900), "bf16")
    q, k, v, sq, sk = prefill_inputs(p)
    qd, kc, vc, skd = decode_inputs(dp)
    o = torch.empty_like(q)
    lse = torch.empty((2, 8, 300), dtype=torch.float32, device=DEV)
    od = torch.empty_like(qd)
    lsed = torch.empty((4, 8), dtype=torch.float32, device=DEV)
    ws = torch.empty(fa.decode_workspace_size(qd, kc, vc), dtype=torch.uint8, device=DEV)

    def calls():
        fa.prefill(q, k, v, causal=True, scale=p.scale, seqlens_q=sq, seqlens_k=sk, out=o, lse=lse)
        fa.decode(qd, kc, vc, skd, scale=dp.scale, out=od, lse=lsed, workspace=ws)

    say("[graph] eager reference")
    calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, od, lsed)]

    say("[graph] capture")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()                                     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, lse, od, lsed):
            t.fill_(float("nan"))                   # eager work between replays
        torch.cuda.synchronize()
        say(f"[graph] replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, lse, od, lsed), ref):
            assert torch.equal(got.view(torch.int32) if got.dtype == torch.float32 else
                               got.view(torch.int16),
                               want.view(torch.int32) if want.dtype == torch.float32 else
                               want.view(torch.int16)), f"replay {rep} differs"


def _check_graph(calls, outs, ctx):
    """Eager reference, capture on a side stream, three replays with eager
    work between them; every replay must match the eager results bit for bit."""
    calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[graph] {ctx} replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            bits = torch.int32 if got.dtype == torch.float32 else torch.int16
            assert torch.equal(got.view(bits), want.view(bits)), f"{ctx}: replay {rep} differs"


def test_persistent_prefill_fp8_decode_and_item_table_in_a_graph():
    """The paths added later in one graph: the persistent packed prefill
    (more work items than CUs), the FP8-cache decode, and a decode of more
    than 64 sequences, whose plan kernel writes the item table into the
    workspace on every replay."""
    from gpu_helpers import dev_tensor, fp8_tensor
    p = workloads.make_prefill(142, 2, 1100, 1100, 32, 8, 128, "bf16", causal=True, window_left=300)
    q, k, v, sq, sk = prefill_inputs(p)
    o = torch.empty_like(q)
    lse = torch.empty((2, 32, 1100), dtype=torch.float32, device=DEV)
    d8 = workloads.make_decode(143, 6, 16, 4, 128, 1200, (1, 1200), "bf16", kv_dtype="fp8_e4m3")
    q8 = dev_tensor(d8.q, d8.dtype)
    k8, v8 = fp8_tensor(d8.k_cache), fp8_tensor(d8.v_cache)
    sk8 = torch.from_numpy(d8.seqlens_k).to(DEV)
    ks, vs = torch.from_numpy(d8.k_scale).to(DEV), torch.from_numpy(d8.v_scale).to(DEV)
    o8 = torch.empty_like(q8)
    l8 = torch.empty((6, 16), dtype=torch.float32, device=DEV)
    ws8 = torch.empty(fa.decode_workspace_size(q8, k8, v8, k_scale=ks, v_scale=vs), dtype=torch.uint8,
                      device=DEV)
    db = workloads.make_decode(144, 80, 8, 2, 128, 600, (1, 600), "bf16")
    qb, kb, vb, skb = decode_inputs(db)
    ob = torch.empty_like(qb)
    lb = torch.empty((80, 8), dtype=torch.float32, device=DEV)
    wsb = torch.empty(fa.decode_workspace_size(qb, kb, vb), dtype=torch.uint8, device=DEV)

    def calls():
        fa.prefill(q, k, v, causal=True, window=300, scale=p.scale, out=o, lse=lse)
        fa.decode(q8, k8, v8, sk8, scale=d8.scale, out=o8, lse=l8, workspace=ws8, k_scale=ks, v_scale=vs)
        fa.decode(qb, kb, vb, skb, scale=db.scale, out=ob, lse=lb, workspace=wsb)

    say("[graph] persistent prefill, FP8 decode, 80-sequence decode")
    _check_graph(calls, (o, lse, o8, l8, ob, lb), "persistent + fp8 + item table")
