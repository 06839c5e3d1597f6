"""GPU check of fa_decode_fwd_noalloc (through the C ABI) against
fa_decode_fwd with a caller workspace: the same kernels on the same inputs,
so the outputs must agree bit for bit (and both sit within the method's bf16
bounds of the fp64 oracle).  Two calls in a row, the second smaller than the
first, so the second runs over the array the first one left filled; neither
call may allocate device memory.
"""
import numpy as np
import pytest
import torch

import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import DEV, check, decode_inputs, oracle_decode, say, to_np

pytestmark = pytest.mark.gpu


def _both(dp, **kw):
    q, kc, vc, sk = decode_inputs(dp)
    B, Hq, d = q.shape
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    fa.decode(q, kc, vc, sk, scale=dp.scale, window=dp.window_left, out=o_ref, lse=l_ref, **kw)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    fa.decode_noalloc(q, kc, vc, sk, scale=dp.scale, window=dp.window_left, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(DEV) == before, "the no-alloc call allocated device memory"
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from fa_decode_fwd"
    assert torch.equal(lse, l_ref), "LSE differs from fa_decode_fwd"
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def test_decode_noalloc_matches_workspace_call_twice():
    # first call: the full decode workload (B64 Hq32 Hkv8 d128, lengths U[512, 8192])
    dp = workloads.make_workload(5)
    ws = fa.decode_workspace_size(*decode_inputs(dp)[:3])
    say(f"[noalloc] call 1: decode B64 Hq32 Hkv8 d128 capacity 8192 (workspace {ws} bytes)")
    o, lse = _both(dp)
    batches = [0, 17, 63]
    ro, rl = oracle_decode(dp, batches=batches)
    check(o[batches], lse[batches], ro, rl, "bf16", "noalloc call 1 (3 sequences)")
    # second call, smaller: fewer sequences, GQA group 2, a window, 128-key chunks
    dp2 = workloads.make_decode(211, 5, 8, 4, 128, 3000, (1, 3000), "bf16", window_left=700)
    say("[noalloc] call 2: decode B5 Hq8 Hkv4 d128 capacity 3000 window 700, chunks of 128")
    o2, l2 = _both(dp2, chunk_keys=128)
    ro2, rl2 = oracle_decode(dp2)
    check(o2, l2, ro2, rl2, "bf16", "noalloc call 2")


def test_decode_noalloc_large_batch_item_table():
    """Above 64 sequences the work-item table also lives in the array."""
    dp = workloads.make_decode(213, 300, 8, 2, 128, 600, (0, 600), "bf16")
    say("[noalloc] decode B300 Hq8 Hkv2 d128 capacity 600 (item table in the array)")
    o, lse = _both(dp)
    ro, rl = oracle_decode(dp)
    check(o, lse, ro, rl, "bf16", "noalloc B300")


def test_decode_noalloc_rejects_oversize():
    """4096 sequences at capacity 1024 in 128-key chunks would need about
    136 MB of partials, beyond the array: refused on the host, before any
    launch, with FA_ERR_WORKSPACE (the cache is one sequence broadcast over
    the batch with a zero stride, so the inputs stay small)."""
    dp = workloads.make_decode(212, 1, 8, 2, 128, 1024, (1, 1024), "bf16")
    q, kc, vc, sk = decode_inputs(dp)
    B = 4096
    big_q = q.expand(B, 8, 128)
    say("[noalloc] oversize request (refused on the host)")
    with pytest.raises(fa.FAError) as ei:
        fa.decode_noalloc(big_q, kc.expand(B, 1024, 2, 128), vc.expand(B, 1024, 2, 128),
                          torch.ones(B, dtype=torch.int32, device=DEV),
                          out=torch.empty((B, 8, 128), dtype=q.dtype, device=DEV),
                          lse=torch.empty((B, 8), device=DEV), chunk_keys=128)
    assert ei.value.status == 3 and "fa_decode_fwd_noalloc" in str(ei.value)
