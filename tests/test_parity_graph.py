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
