"""Writes tests/golden/tiny_bf16_oracle.json from the oracle alone.

The pages print no worked numeric example for this method, so the stored
values here are the oracle's own float64 result on the seeded tiny workload
(B=2, H=16, seq_lens [37, 100], page size 32, bmm1 1/sqrt(192), bmm2 1).  It
is a regression fixture for the generator + oracle pair: a change to either
that moves these numbers must be deliberate.  Run: python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from paged_mla_decode_03_amd.inputs import named_workload  # noqa: E402


def main():
    w = named_workload("tiny_bf16")
    out, lse = oracle.reference_decode(oracle.MlaProblem(**w.oracle_problem_kwargs()))
    data = {
        "workload": "tiny_bf16 (seed 1)",
        "source": "oracle/mla.py reference_decode, float64",
        "lse": [[float(v) for v in row] for row in lse.reshape(-1, 16)],
        "out_first8": [[[float(v) for v in out[r, h, :8]] for h in range(16)] for r in range(out.shape[0])],
        "out_row_sums": [[float(out[r, h].sum()) for h in range(16)] for r in range(out.shape[0])],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_bf16_oracle.json")
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
