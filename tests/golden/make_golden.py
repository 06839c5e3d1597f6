"""Writes tests/golden/input_hashes.json: SHA-256 of generated input bytes.

Calls only the seeded input generators (``workloads``); the hashes pin the
generator so that the oracle and the GPU path keep seeing the same bits on
every machine.  Run from the repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402


def main():
    out = {
        "workload_1": workloads.make_workload(1).sha256(),
        "prefill_small": workloads.make_prefill(5, 2, 70, 70, 4, 2, 64, "bf16", causal=True,
                                                seqlens_k_range=(1, 70)).sha256(),
        "decode_small": workloads.make_decode(6, 3, 4, 2, 64, 300, (1, 300), "bf16").sha256(),
        "decode_paged_small": workloads.make_decode_paged(6, 3, 4, 2, 64, 300, (1, 300), 16,
                                                          "bf16").sha256(),
        "decode_fp8_small": workloads.make_decode(6, 3, 4, 2, 64, 300, (1, 300), "bf16",
                                                  kv_dtype="fp8_e4m3").sha256(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_hashes.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
