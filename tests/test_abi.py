"""C-ABI checks that need no GPU.

* the shared library loads and exports every function ``include/fa.h``
  declares;
* the ctypes structs match the C layout (sizes and offsets from a program
  compiled with gcc against the header);
* every argument check returns its status and message before any HIP call
  (none of these cases reaches a launch);
* the decode workspace size is a host-side formula.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from transformer_attention_flashattention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfa.so is not built: run __graft_entry__.build() first")
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared:
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_abi_version_and_status_strings(lib):
    m = re.search(r"#define FA_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.fa_abi_version() == int(m.group(1))
    names = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED",
             3: "FA_ERR_WORKSPACE", 4: "FA_ERR_HIP"}
    for code, name in names.items():
        assert _lib.status_str(code) == name
    assert _lib.status_str(99) == "FA_ERR_UNKNOWN"


LAYOUT_PROG = r"""
#include <stdio.h>
#include <stddef.h>
#include "fa.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("prefill %zu\n", sizeof(fa_prefill_params));
  printf("decode %zu\n", sizeof(fa_decode_params));
  F(fa_prefill_params, softmax_scale) F(fa_prefill_params, q) F(fa_prefill_params, lse)
  F(fa_prefill_params, seqlens_k) F(fa_prefill_params, q_stride) F(fa_prefill_params, o_stride)
  F(fa_decode_params, softmax_scale) F(fa_decode_params, reserved0) F(fa_decode_params, q)
  F(fa_decode_params, seqlens_k) F(fa_decode_params, q_stride) F(fa_decode_params, k_stride)
  F(fa_decode_params, o_stride) F(fa_prefill_params, alibi_slopes) F(fa_decode_params, alibi_slopes)
  F(fa_decode_params, block_table) F(fa_decode_params, page_size) F(fa_decode_params, pages_per_seq)
  F(fa_decode_params, num_pages) F(fa_decode_params, reserved1) F(fa_decode_params, kv_format)
  F(fa_decode_params, reserved2) F(fa_decode_params, k_scale) F(fa_decode_params, v_scale)
  F(fa_decode_params, rope_cos) F(fa_decode_params, rope_sin) F(fa_decode_params, rotary_dim)
  F(fa_decode_params, rope_max_pos) F(fa_prefill_params, rope_cos) F(fa_prefill_params, rope_sin)
  F(fa_prefill_params, rotary_dim) F(fa_prefill_params, rope_max_pos)
  F(fa_prefill_params, workspace) F(fa_prefill_params, workspace_bytes)
  F(fa_prefill_params, attn_mask) F(fa_prefill_params, mask_stride)
  return 0;
}
"""


def test_struct_layout_matches_c():
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "layout.c")
        exe = os.path.join(td, "layout")
        open(src, "w").write(LAYOUT_PROG)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), src,
                        "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    vals = dict(line.rsplit(" ", 1) for line in out.splitlines())
    assert int(vals["prefill"]) == ctypes.sizeof(_lib.PrefillParams)
    assert int(vals["decode"]) == ctypes.sizeof(_lib.DecodeParams)
    for key, v in vals.items():
        if "." not in key:
            continue
        struct, field = key.split(".")
        cls = _lib.PrefillParams if struct == "fa_prefill_params" else _lib.DecodeParams
        assert getattr(cls, field).offset == int(v), key


# ---------------------------------------------------------------------------
# Validation: each case must fail on the host, before any HIP call.
# Pointers are fake (never dereferenced) but 16-byte aligned unless the case
# is about alignment.
# ---------------------------------------------------------------------------
FAKE = 0x10000


def _prefill(**kw):
    p = _lib.PrefillParams()
    p.dtype = _lib.FA_DTYPE_BF16
    p.batch, p.seqlen_q, p.seqlen_k = 2, 100, 100
    p.heads_q, p.heads_kv, p.head_dim = 8, 2, 128
    p.causal, p.window_left, p.softmax_scale = 1, -1, 0.088
    p.q, p.k, p.v, p.o, p.lse = FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, FAKE + 16384
    st = [100 * 8 * 128, 8 * 128, 128]
    stk = [100 * 2 * 128, 2 * 128, 128]
    p.q_stride[:] = st
    p.k_stride[:] = stk
    p.v_stride[:] = stk
    p.o_stride[:] = st
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(p, k)[:] = v
        else:
            setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=7), _lib.FA_ERR_INVALID_ARG, "dtype"),
    (dict(batch=-1), _lib.FA_ERR_INVALID_ARG, "batch"),
    (dict(heads_kv=3), _lib.FA_ERR_INVALID_ARG, "multiple"),
    (dict(heads_q=0), _lib.FA_ERR_INVALID_ARG, "heads"),
    (dict(head_dim=96), _lib.FA_ERR_UNSUPPORTED, "head_dim"),
    (dict(window_left=0), _lib.FA_ERR_INVALID_ARG, "window"),
    (dict(window_left=-5), _lib.FA_ERR_INVALID_ARG, "window"),
    (dict(causal=2), _lib.FA_ERR_INVALID_ARG, "causal"),
    (dict(softmax_scale=0.0), _lib.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(softmax_scale=float("nan")), _lib.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(softmax_scale=-0.1), _lib.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(q_stride=[100 * 8 * 128, 8 * 128, 130]), _lib.FA_ERR_UNSUPPORTED, "q_stride"),
    (dict(k_stride=[-1, 256, 128]), _lib.FA_ERR_INVALID_ARG, "k_stride"),
    (dict(q=None), _lib.FA_ERR_INVALID_ARG, "non-NULL"),
    (dict(v=None), _lib.FA_ERR_INVALID_ARG, "non-NULL"),
    (dict(o=FAKE + 2), _lib.FA_ERR_UNSUPPORTED, "aligned"),
    (dict(k_stride=[1 << 30, 1 << 25, 128]), _lib.FA_ERR_UNSUPPORTED, "2^25"),
    (dict(v_stride=[1 << 30, 1 << 25, 128]), _lib.FA_ERR_UNSUPPORTED, "2^25"),
    # RoPE
    (dict(rotary_dim=4, rope_max_pos=100), _lib.FA_ERR_UNSUPPORTED, "rotary_dim"),
    (dict(rotary_dim=136, rope_max_pos=100), _lib.FA_ERR_UNSUPPORTED, "rotary_dim"),
    (dict(rotary_dim=-8, rope_max_pos=100), _lib.FA_ERR_UNSUPPORTED, "rotary_dim"),
    (dict(rotary_dim=64, rope_max_pos=99), _lib.FA_ERR_INVALID_ARG, "rope_max_pos"),
    (dict(rotary_dim=64, rope_max_pos=100, rope_cos=None, rope_sin=FAKE + 32768),
     _lib.FA_ERR_INVALID_ARG, "rope_cos"),
    (dict(rotary_dim=64, rope_max_pos=100, rope_cos=FAKE + 28680, rope_sin=FAKE + 32768),
     _lib.FA_ERR_UNSUPPORTED, "16-byte"),
    (dict(rotary_dim=64, rope_max_pos=100, rope_cos=FAKE + 28672, rope_sin=FAKE + 32768),
     _lib.FA_ERR_WORKSPACE, "workspace is NULL"),
    (dict(rotary_dim=64, rope_max_pos=100, rope_cos=FAKE + 28672, rope_sin=FAKE + 32768,
          workspace=FAKE + 65536, workspace_bytes=2 * 100 * 2 * 128 * 2 - 1),
     _lib.FA_ERR_WORKSPACE, "too small"),
    (dict(rotary_dim=64, rope_max_pos=100, rope_cos=FAKE + 28672, rope_sin=FAKE + 32768,
          workspace=FAKE + 65544, workspace_bytes=1 << 30), _lib.FA_ERR_WORKSPACE, "aligned"),
    # explicit mask
    (dict(attn_mask=FAKE + 40960, mask_stride=[100, 0, 0, 0]), _lib.FA_ERR_UNSUPPORTED,
     "mask_stride[3]"),
    (dict(attn_mask=FAKE + 40960, mask_stride=[100, 0, 0, 1]), _lib.FA_ERR_UNSUPPORTED,
     "mask_stride[0]"),
    (dict(attn_mask=FAKE + 40960, mask_stride=[104, 0, -8, 1]), _lib.FA_ERR_INVALID_ARG,
     "mask_stride[2]"),
    (dict(attn_mask=FAKE + 40962, mask_stride=[104, 0, 0, 1]), _lib.FA_ERR_UNSUPPORTED,
     "attn_mask must be 16-byte aligned"),
])
def test_prefill_validation(lib, kw, status, needle):
    p = _prefill(**kw)
    st = _lib.prefill_fwd(p, 0)
    assert st == status, (_lib.status_str(st), _lib.last_error())
    assert needle in _lib.last_error()


def test_prefill_workspace_size(lib):
    # only bf16 with RoPE needs a workspace: the rotated copy of K
    assert _lib.prefill_workspace_size(_prefill()) == (_lib.FA_OK, 0)
    p = _prefill(rotary_dim=64, rope_max_pos=100)
    assert _lib.prefill_workspace_size(p) == (_lib.FA_OK, 2 * 100 * 2 * 128 * 2)
    p = _prefill(dtype=_lib.FA_DTYPE_F32, rotary_dim=64, rope_max_pos=100)
    assert _lib.prefill_workspace_size(p) == (_lib.FA_OK, 0)
    p = _prefill(dtype=_lib.FA_DTYPE_F16, rotary_dim=64, rope_max_pos=100)
    assert _lib.prefill_workspace_size(p) == (_lib.FA_OK, 2 * 100 * 2 * 128 * 2)
    p = _prefill(rotary_dim=12, rope_max_pos=100)
    assert _lib.prefill_workspace_size(p)[0] == _lib.FA_ERR_UNSUPPORTED
    p = _prefill(batch=70000, rotary_dim=64, rope_max_pos=100)
    assert _lib.prefill_workspace_size(p)[0] == _lib.FA_ERR_UNSUPPORTED
    assert "65535" in _lib.last_error()


def test_prefill_fp32_stride_rule(lib):
    # fp32 needs strides in multiples of 4 elements, bf16 in multiples of 8
    p = _prefill(dtype=_lib.FA_DTYPE_F32, q_stride=[100 * 8 * 128, 8 * 128, 130])
    assert _lib.prefill_fwd(p, 0) == _lib.FA_ERR_UNSUPPORTED
    p = _prefill(dtype=_lib.FA_DTYPE_F32, q_stride=[100 * 8 * 128, 8 * 128, 132], q=None)
    assert _lib.prefill_fwd(p, 0) == _lib.FA_ERR_INVALID_ARG
    p = _prefill(dtype=_lib.FA_DTYPE_BF16, q_stride=[100 * 8 * 128, 8 * 128, 132])
    assert _lib.prefill_fwd(p, 0) == _lib.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(batch=0), dict(seqlen_q=0)])
def test_prefill_empty_is_noop(lib, kw):
    # no launch happens for an empty problem, so fake pointers are fine
    p = _prefill(**kw)
    assert _lib.prefill_fwd(p, 0) == _lib.FA_OK
    assert _lib.last_error() == ""


def _decode(**kw):
    p = _lib.DecodeParams()
    p.dtype = _lib.FA_DTYPE_BF16
    p.batch, p.heads_q, p.heads_kv, p.head_dim = 64, 32, 8, 128
    p.cache_capacity, p.window_left, p.chunk_keys = 8192, -1, 0
    p.softmax_scale, p.reserved0 = 0.088, 0
    p.q, p.k_cache, p.v_cache, p.o, p.lse, p.seqlens_k = (FAKE, FAKE + 4096, FAKE + 8192,
                                                          FAKE + 12288, FAKE + 16384, FAKE + 20480)
    p.q_stride[:] = [32 * 128, 128]
    p.k_stride[:] = [8192 * 8 * 128, 8 * 128, 128]
    p.v_stride[:] = [8192 * 8 * 128, 8 * 128, 128]
    p.o_stride[:] = [32 * 128, 128]
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(p, k)[:] = v
        else:
            setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=_lib.FA_DTYPE_F32), _lib.FA_ERR_UNSUPPORTED, "bf16"),
    (dict(dtype=3), _lib.FA_ERR_INVALID_ARG, "dtype"),
    (dict(heads_kv=5), _lib.FA_ERR_INVALID_ARG, "multiple"),
    (dict(head_dim=80), _lib.FA_ERR_UNSUPPORTED, "head_dim"),
    (dict(cache_capacity=0), _lib.FA_ERR_INVALID_ARG, "capacity"),
    (dict(window_left=0), _lib.FA_ERR_INVALID_ARG, "window"),
    (dict(chunk_keys=100), _lib.FA_ERR_UNSUPPORTED, "chunk_keys"),
    (dict(chunk_keys=64), _lib.FA_ERR_UNSUPPORTED, "chunk_keys"),
    (dict(chunk_keys=-128), _lib.FA_ERR_UNSUPPORTED, "chunk_keys"),
    (dict(chunk_keys=65536 + 128), _lib.FA_ERR_UNSUPPORTED, "chunk_keys"),
    (dict(reserved0=1), _lib.FA_ERR_INVALID_ARG, "reserved0"),
    (dict(reserved1=1), _lib.FA_ERR_INVALID_ARG, "reserved1"),
    (dict(reserved2=1), _lib.FA_ERR_INVALID_ARG, "reserved2"),
    # FP8 cache format
    (dict(kv_format=2), _lib.FA_ERR_INVALID_ARG, "kv_format"),
    (dict(k_scale=FAKE + 28672), _lib.FA_ERR_INVALID_ARG, "FA_KV_PLAIN"),
    (dict(kv_format=1, k_scale=FAKE + 28672, v_scale=FAKE + 28800,
          k_stride=[8192 * 8 * 128, 8 * 128 + 8, 128]), _lib.FA_ERR_UNSUPPORTED, "k_stride"),
    (dict(kv_format=1, k_scale=None, v_scale=FAKE + 28800), _lib.FA_ERR_INVALID_ARG, "non-NULL"),
    (dict(kv_format=1, k_scale=FAKE + 28674, v_scale=FAKE + 28800), _lib.FA_ERR_INVALID_ARG,
     "4-byte aligned"),
    (dict(rotary_dim=12, rope_max_pos=8192), _lib.FA_ERR_UNSUPPORTED, "rotary_dim"),
    (dict(rotary_dim=64, rope_max_pos=8191), _lib.FA_ERR_INVALID_ARG, "rope_max_pos"),
    (dict(rotary_dim=64, rope_max_pos=8192, rope_cos=FAKE + 28680, rope_sin=FAKE + 32768),
     _lib.FA_ERR_UNSUPPORTED, "16-byte"),
    # paged-cache fields without a table, and bad paged parameters
    (dict(page_size=16), _lib.FA_ERR_INVALID_ARG, "without a block_table"),
    (dict(num_pages=4), _lib.FA_ERR_INVALID_ARG, "without a block_table"),
    (dict(block_table=FAKE + 24576, page_size=8, pages_per_seq=1024, num_pages=100),
     _lib.FA_ERR_UNSUPPORTED, "page_size"),
    (dict(block_table=FAKE + 24576, page_size=24, pages_per_seq=512, num_pages=100),
     _lib.FA_ERR_UNSUPPORTED, "page_size"),
    (dict(block_table=FAKE + 24576, page_size=65536 + 16, pages_per_seq=1, num_pages=100),
     _lib.FA_ERR_UNSUPPORTED, "page_size"),
    (dict(block_table=FAKE + 24576, page_size=16, pages_per_seq=0, num_pages=100),
     _lib.FA_ERR_INVALID_ARG, "pages_per_seq"),
    (dict(block_table=FAKE + 24576, page_size=16, pages_per_seq=512, num_pages=0),
     _lib.FA_ERR_INVALID_ARG, "num_pages"),
    (dict(block_table=FAKE + 24576, page_size=16, pages_per_seq=511, num_pages=100),
     _lib.FA_ERR_INVALID_ARG, "exceeds pages_per_seq"),
    (dict(block_table=FAKE + 24578, page_size=16, pages_per_seq=512, num_pages=100),
     _lib.FA_ERR_INVALID_ARG, "4-byte"),
    (dict(softmax_scale=float("inf")), _lib.FA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(seqlens_k=None), _lib.FA_ERR_INVALID_ARG, "seqlens_k"),
    (dict(k_cache=FAKE + 8), _lib.FA_ERR_UNSUPPORTED, "aligned"),
    (dict(k_stride=[8192 * 8 * 128, 8 * 128, 132]), _lib.FA_ERR_UNSUPPORTED, "k_stride"),
])
def test_decode_validation(lib, kw, status, needle):
    p = _decode(**kw)
    st = _lib.decode_fwd(p, FAKE, 1 << 40, 0)
    assert st == status, (_lib.status_str(st), _lib.last_error())
    assert needle in _lib.last_error()
    st2, _ = _lib.decode_workspace_size(p)
    if needle in ("seqlens_k", "aligned", "4-byte", "non-NULL", "4-byte aligned", "16-byte"):
        # sizing the workspace needs shapes only, never the data pointers
        assert st2 == _lib.FA_OK
    else:
        assert st2 == status


def test_decode_noalloc_validation_before_any_hip_call(lib):
    """fa_decode_fwd_noalloc runs the decode's argument checks, then refuses
    a problem whose workspace would not fit its FA_DECODE_NOALLOC_MAX_BYTES
    device array, all before touching the GPU (none of these reaches a HIP
    call, so they run here without one)."""
    m = re.search(r"#define FA_DECODE_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == _lib.DECODE_NOALLOC_MAX_BYTES
    for kw, status, needle in [(dict(head_dim=80), _lib.FA_ERR_UNSUPPORTED, "head_dim"),
                               (dict(seqlens_k=None), _lib.FA_ERR_INVALID_ARG, "seqlens_k"),
                               (dict(window_left=0), _lib.FA_ERR_INVALID_ARG, "window")]:
        assert _lib.decode_fwd_noalloc(_decode(**kw), 0) == status
        assert needle in _lib.last_error()
    # 64 x 32 heads at capacity 8192 in 128-key chunks: 8.5 MiB x 64 / 4 > 32 MiB
    big = _decode(chunk_keys=128)
    st, need = _lib.decode_workspace_size(big)
    assert st == _lib.FA_OK and need > _lib.DECODE_NOALLOC_MAX_BYTES
    assert _lib.decode_fwd_noalloc(big, 0) == _lib.FA_ERR_WORKSPACE
    assert "fa_decode_fwd_noalloc" in _lib.last_error() and str(need) in _lib.last_error()
    # an empty batch is a no-op
    assert _lib.decode_fwd_noalloc(_decode(batch=0), 0) == _lib.FA_OK


def test_decode_rejects_cache_rows_beyond_32bit_offsets(lib):
    # the split kernel addresses one sequence's rows with 32-bit byte offsets
    p = _decode(batch=1, cache_capacity=1 << 22,
                k_stride=[(1 << 22) * 8 * 128, 8 * 128, 128],
                v_stride=[(1 << 22) * 8 * 128, 8 * 128, 128])
    assert _lib.decode_fwd(p, FAKE, 1 << 40, 0) == _lib.FA_ERR_UNSUPPORTED
    assert "4 GiB" in _lib.last_error()
    p = _decode(batch=1, cache_capacity=1 << 20,
                k_stride=[(1 << 20) * 8 * 128, 8 * 128, 128],
                v_stride=[(1 << 20) * 8 * 128, 8 * 128, 128])
    st, n = _lib.decode_workspace_size(p)
    assert st == _lib.FA_OK and n > 0


def test_decode_workspace_rules(lib):
    p = _decode()
    st, n = _lib.decode_workspace_size(p)
    assert st == _lib.FA_OK
    # library choice at this size is 2048-key chunks: 4 chunks of 64*32 rows
    rows = 64 * 32 * 4
    expect = ((rows * 128 * 4 + 255) // 256) * 256 + rows * 2 * 4
    assert n == expect
    assert _lib.decode_fwd(p, None, n, 0) == _lib.FA_ERR_WORKSPACE
    assert "NULL" in _lib.last_error()
    assert _lib.decode_fwd(p, FAKE, n - 1, 0) == _lib.FA_ERR_WORKSPACE
    assert "too small" in _lib.last_error()
    assert _lib.decode_fwd(p, FAKE + 4, n, 0) == _lib.FA_ERR_WORKSPACE
    # explicit chunk sizes change the requirement accordingly
    p128 = _decode(chunk_keys=128)
    _, n128 = _lib.decode_workspace_size(p128)
    rows = 64 * 32 * 64
    assert n128 == ((rows * 128 * 4 + 255) // 256) * 256 + rows * 2 * 4
    # a small batch at low capacity gets shorter chunks (more workgroups)
    ps = _decode(batch=2, cache_capacity=1000)
    _, ns = _lib.decode_workspace_size(ps)
    rows = 2 * 32 * 8          # 16 kv groups x ceil(1000/128) < 4096 -> 128-key chunks
    assert ns == ((rows * 128 * 4 + 255) // 256) * 256 + rows * 2 * 4
    # empty batch is a no-op needing no workspace
    p0 = _decode(batch=0)
    assert _lib.decode_workspace_size(p0) == (_lib.FA_OK, 0)
    assert _lib.decode_fwd(p0, None, 0, 0) == _lib.FA_OK


def test_no_unresolved_internal_symbols(lib):
    """Every kernel launcher links: a kernel whose host-side instantiation fails
    leaves an undefined device stub behind, which only shows at load time."""
    out = subprocess.run(["nm", "-D", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    undefined = [l.split()[-1] for l in out.splitlines() if l.strip().startswith("U ")]
    assert not [s for s in undefined if s.startswith("_ZN2fa")], undefined


def test_decode_paged_limits(lib):
    # paged: only one page's rows need 32-bit offsets, not the whole capacity
    pg = dict(block_table=FAKE + 24576, page_size=256, num_pages=1 << 16)
    p = _decode(batch=1, cache_capacity=1 << 22, pages_per_seq=(1 << 22) // 256,
                k_stride=[256 * 8 * 128, 8 * 128, 128], v_stride=[256 * 8 * 128, 8 * 128, 128], **pg)
    st, n = _lib.decode_workspace_size(p)
    assert st == _lib.FA_OK and n > 0
    # a page whose rows need more than 32-bit offsets is refused
    p = _decode(batch=1, cache_capacity=65536, page_size=65536, pages_per_seq=1,
                block_table=FAKE + 24576, num_pages=2,
                k_stride=[65536 * 65536, 65536, 128], v_stride=[65536 * 65536, 65536, 128])
    assert _lib.decode_fwd(p, FAKE, 1 << 40, 0) == _lib.FA_ERR_UNSUPPORTED
    assert "per page" in _lib.last_error()
    # the table's entry count must fit int32
    p = _decode(batch=64, cache_capacity=8192, page_size=16, pages_per_seq=1 << 26,
                block_table=FAKE + 24576, num_pages=2)
    assert _lib.decode_workspace_size(p)[0] == _lib.FA_ERR_UNSUPPORTED
    assert "2^31" in _lib.last_error()
    # the workspace depends on the logical capacity only, paged or not
    plain = _lib.decode_workspace_size(_decode())
    paged = _lib.decode_workspace_size(_decode(block_table=FAKE + 24576, page_size=16,
                                               pages_per_seq=512, num_pages=40000,
                                               k_stride=[16 * 8 * 128, 8 * 128, 128],
                                               v_stride=[16 * 8 * 128, 8 * 128, 128]))
    assert plain == paged


def test_decode_fp8_strides_and_offsets(lib):
    # FP8 codes are one byte: a stride of 16 elements is enough, 8 is not
    base = dict(kv_format=1, k_scale=FAKE + 28672, v_scale=FAKE + 28800)
    p = _decode(k_stride=[8192 * 8 * 128, 8 * 128 + 16, 128], **base)
    assert _lib.decode_workspace_size(p)[0] == _lib.FA_OK
    p = _decode(k_stride=[8192 * 8 * 128, 8 * 128 + 8, 128], **base)
    assert _lib.decode_workspace_size(p)[0] == _lib.FA_ERR_UNSUPPORTED
    # the 32-bit row offsets count bytes: 2^22 rows of 1 KiB codes fit, the same
    # rows in bf16 would not
    big = dict(batch=1, cache_capacity=1 << 22, k_stride=[(1 << 22) * 1024, 1024, 128],
               v_stride=[(1 << 22) * 1024, 1024, 128])
    assert _lib.decode_fwd(_decode(**big), FAKE, 1 << 40, 0) == _lib.FA_ERR_UNSUPPORTED
    assert "4 GiB" in _lib.last_error()
    st, n = _lib.decode_workspace_size(_decode(**big, **base))
    assert st == _lib.FA_OK and n > 0


def test_half_dtype_rules(lib):
    # half takes the 16-bit rules: strides in multiples of 8 elements, seq
    # strides below 2^25; decode accepts it, and fp32 decode stays unsupported
    p = _prefill(dtype=_lib.FA_DTYPE_F16, q_stride=[100 * 8 * 128, 8 * 128, 132])
    assert _lib.prefill_fwd(p, 0) == _lib.FA_ERR_UNSUPPORTED
    p = _prefill(dtype=_lib.FA_DTYPE_F16, k_stride=[1 << 30, 1 << 25, 128])
    assert _lib.prefill_fwd(p, 0) == _lib.FA_ERR_UNSUPPORTED and "2^25" in _lib.last_error()
    assert _lib.decode_workspace_size(_decode(dtype=_lib.FA_DTYPE_F16))[0] == _lib.FA_OK
    assert _lib.decode_workspace_size(_decode(dtype=_lib.FA_DTYPE_F32))[0] == _lib.FA_ERR_UNSUPPORTED
    assert _lib.decode_workspace_size(_decode(dtype=3))[0] == _lib.FA_ERR_INVALID_ARG
