"""GPU parity: fa_decode_fwd over a paged KV cache (block table into a page
pool) against the fp64 oracle's gather-then-decode.  The pools come from the
generator: pages in a seeded random order, NaN in every slot past a
sequence's length, in the spare page, and behind every table entry past the
pages in use, so a read the lengths do not allow poisons the output.
"""
import numpy as np
import pytest
import torch

import transformer_attention_flashattention_amd as fa
import workloads
from gpu_helpers import (DEV, check, decode_inputs, oracle_decode_paged, paged_inputs,
                         run_decode_paged, say, to_np)

pytestmark = pytest.mark.gpu


def _case(pp, ctx, alibi_slopes=None, **kw):
    say(f"[paged] {ctx} B={pp.q.shape[0]} Hq={pp.q.shape[1]} Hkv={pp.k_pool.shape[2]} "
        f"d={pp.q.shape[2]} page={pp.page_size} pages={pp.k_pool.shape[0]} "
        f"cap={pp.capacity} W={pp.window_left} {kw}")
    o, lse = run_decode_paged(pp, alibi_slopes=alibi_slopes, **kw)
    ro, rl = oracle_decode_paged(pp, alibi_slopes=alibi_slopes)
    check(o, lse, ro, rl, pp.dtype, ctx)
    return o, lse


@pytest.mark.parametrize("page", [16, 256])
def test_paged_decode_workload_shape(page):
    """The decode workload (B64 Hq32 Hkv8 d128, L ~ U[512, 8192]) in a paged pool."""
    pp = workloads.make_decode_paged(5, 64, 32, 8, 128, 8192, (512, 8192), page, "bf16")
    _case(pp, f"decode workload, page {page}")


@pytest.mark.parametrize("page", [16, 64, 256])
@pytest.mark.parametrize("chunk", [0, 128])
def test_paged_bit_identical_to_contiguous(page, chunk):
    """Same logical cache (same seed) in both layouts, no window: the kernels
    visit the same keys in the same order, so the outputs agree bit for bit."""
    lengths = np.array([1, 15, 16, 17, 300, 1024, 0, 999], dtype=np.int32)
    dp = workloads.make_decode(60, 8, 8, 2, 128, 1024, (1, 1024), "bf16", lengths=lengths)
    pp = workloads.make_decode_paged(60, 8, 8, 2, 128, 1024, (1, 1024), page, "bf16",
                                     lengths=lengths)
    say(f"[paged] bitwise vs contiguous page={page} chunk={chunk}")
    q, kc, vc, sk = decode_inputs(dp)
    o1, l1 = fa.decode(q, kc, vc, sk, scale=dp.scale, chunk_keys=chunk)
    q, kp, vp, sk, table = paged_inputs(pp)
    o2, l2 = fa.decode(q, kp, vp, sk, scale=pp.scale, chunk_keys=chunk, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("page", [16, 32, 48, 128, 272, 1024])
def test_paged_page_sizes_and_edges(page):
    lengths = np.array([1, 15, 16, 17, 47, 48, 49, 127, 128, 129, 271, 272, 273, 600, 0, 1100],
                       dtype=np.int32)
    pp = workloads.make_decode_paged(61, len(lengths), 8, 2, 128, 1100, (1, 1100), page, "bf16",
                                     lengths=lengths, spare_pages=3)
    _case(pp, f"page {page} lengths at page and tile edges")
    _case(pp, f"page {page} lengths at page and tile edges, 128-key chunks", chunk_keys=128)


@pytest.mark.parametrize("W", [1, 17, 100, 1000])
@pytest.mark.parametrize("page", [16, 48])
def test_paged_window(W, page):
    """Windows start at any key, so the first tile of a sequence straddles
    keys the window hides."""
    pp = workloads.make_decode_paged(62, 7, 8, 2, 128, 1300, (1, 1300), page, "bf16",
                                     window_left=W)
    _case(pp, f"window {W}")
    _case(pp, f"window {W}, 128-key chunks", chunk_keys=128)


def test_paged_gqa_d64_alibi():
    pp = workloads.make_decode_paged(63, 5, 12, 4, 64, 900, (1, 900), 32, "bf16")
    slopes = np.linspace(0.01, 0.3, 12).astype(np.float32)
    _case(pp, "d64 GQA 3")
    _case(pp, "d64 GQA 3 ALiBi", alibi_slopes=slopes)
    pp = workloads.make_decode_paged(64, 4, 8, 1, 128, 700, (1, 700), 16, "bf16", window_left=50)
    _case(pp, "MQA window 50 ALiBi", alibi_slopes=np.full(8, 0.05, dtype=np.float32))


def test_paged_unused_entries_and_capacity():
    """Table entries past the pages a sequence uses are never read (they hold
    values outside the pool here), and lengths clamp to the given capacity."""
    pp = workloads.make_decode_paged(65, 4, 8, 2, 128, 512, (1, 512), 16, "bf16",
                                     lengths=np.array([5, 100, 0, 512], dtype=np.int32))
    for b in range(4):
        used = -(-int(pp.seqlens_k[b]) // 16)
        pp.block_table[b, used:] = [(1 << 30) if (i % 2) else -7
                                    for i in range(pp.block_table.shape[1] - used)]
    _case(pp, "garbage past the used pages")
    # capacity below pages_per_seq * page_size: sequence 3 is cut to 300 keys
    q, kp, vp, sk, table = paged_inputs(pp)
    o, lse = fa.decode(q, kp, vp, sk, scale=pp.scale, block_table=table, capacity=300)
    torch.cuda.synchronize()
    ro, rl = oracle_decode_paged(pp, capacity=300)
    check(to_np(o), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", "capacity 300")


def test_paged_out_of_range_entry_is_clamped():
    """An entry outside [0, num_pages) reads the nearest valid page instead of
    leaving the pool; the result is the decode over the clamped table."""
    pp = workloads.make_decode_paged(66, 2, 4, 1, 128, 256, (1, 256), 16, "bf16",
                                     lengths=np.array([40, 200], dtype=np.int32), spare_pages=1)
    n = pp.k_pool.shape[0]
    # the clamped targets must hold finite rows for the comparison: use in-use pages
    pp.block_table[0, 1] = n + 1000          # clamps to n - 1
    pp.block_table[1, 3] = -5                # clamps to 0
    clamped = pp.block_table.copy()
    clamped[0, 1] = n - 1
    clamped[1, 3] = 0
    # make both clamp targets ordinary in-use pages with finite rows
    for phys in (0, n - 1):
        pp.k_pool[phys] = workloads.f32_to_bf16_bits(np.full(pp.k_pool.shape[1:], 0.25, np.float32))
        pp.v_pool[phys] = workloads.f32_to_bf16_bits(
            np.random.default_rng(phys).standard_normal(pp.v_pool.shape[1:], dtype=np.float32))
    o, lse = run_decode_paged(pp)
    ref = workloads.PagedDecodeProblem(pp.dtype, pp.q, pp.k_pool, pp.v_pool, clamped,
                                       pp.seqlens_k, pp.scale)
    ro, rl = oracle_decode_paged(ref)
    check(o, lse, ro, rl, "bf16", "clamped table entries")
