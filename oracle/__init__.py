"""fp64 CPU oracle for the fused-attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import anything under ``oracle/``.  The library's product path
(the C ABI in ``include/fa.h`` and its Python binding) never calls it, and
the two share no code.
"""
from .attention import (alibi_bias, attention, decode, decode_paged, dequantize_kv,  # noqa: F401
                        fp8_e4m3_value, gather_paged, rope_rotate, round_to_dtype, visible,
                        visible_matrix)
