"""Parity report of the GPU path against the oracle on the five workloads.

    python tests/parity_report.py > report.md      (needs a gfx950 GPU)

The table is made by the same comparison that test_workload_full_size
asserts on (tests/test_gpu_parity.py, full_size_parity): every code, scale,
weight code, int32 accumulator and bf16 output of each workload at full
size, through the product path (W8A8Linear), against the oracle; plus the
rel-L2 of the outputs against fp64 matmuls of the dequantized operands (the
pages' 0.17 % statistic) and of the raw bf16 X and fp32 W (the quantization
error). Prints one markdown table.
"""
from __future__ import annotations

import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from tests.test_gpu_parity import PARITY_TABLE_HEAD, full_size_parity, parity_table_row  # noqa: E402
from w8a8_int8_dynamic_amd import ops  # noqa: E402


def main() -> int:
    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 1
    orc = oracle.load()
    print(PARITY_TABLE_HEAD)
    for w in wl.WORKLOADS:
        print(parity_table_row(full_size_parity(ops, orc, w)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
