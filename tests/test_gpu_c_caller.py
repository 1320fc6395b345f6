"""GPU test of the C ABI from a plain C++ program (tests/c_caller/mla_c_caller,
linked by the build step): HIP runtime calls and include/mla_decode.h only, no
Python or torch on the call path.  The test writes a seeded workload to a
folder, runs the program on it, and checks its outputs against the float64
oracle and bitwise against the Python binding's call of the same library."""

import os
import subprocess

import numpy as np
import pytest
import torch

from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, named_workload, INV_SQRT_192

from gpu_cases import check_close, oracle_rows, run_hip

pytestmark = pytest.mark.gpu

CALLER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_caller", "mla_c_caller")


def _run_caller(w, folder):
    assert os.path.exists(CALLER), "tests/c_caller/mla_c_caller is missing: run __graft_entry__.build() first"
    B, H, SQ = w.batch, w.num_heads, w.q_len_fixed
    num_pages, ps = w.kv_bits.shape[0], w.kv_bits.shape[1]
    with open(os.path.join(folder, "meta.txt"), "w") as f:
        f.write(f"{B} {H} {SQ} {ps} {num_pages} {w.block_tables.shape[1]} {w.max_seq_len} {int(w.causal)} "
                f"{float(np.float32(w.bmm1_scale))!r} {float(np.float32(w.bmm2_scale))!r}\n")
    np.ascontiguousarray(w.q_bits, dtype=np.uint16).tofile(os.path.join(folder, "q.bin"))
    np.ascontiguousarray(w.kv_bits, dtype=np.uint16).tofile(os.path.join(folder, "kv.bin"))
    np.ascontiguousarray(w.block_tables, dtype=np.int32).tofile(os.path.join(folder, "bt.bin"))
    np.ascontiguousarray(w.seq_lens, dtype=np.int32).tofile(os.path.join(folder, "lens.bin"))
    print("running the C caller on", w.name, flush=True)
    r = subprocess.run([CALLER, folder], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    out = np.fromfile(os.path.join(folder, "out.bin"), dtype=np.uint16).reshape(w.total_q, H, 512)
    lse = np.fromfile(os.path.join(folder, "lse.bin"), dtype=np.float32).reshape(w.total_q, H)
    out = (out.astype(np.uint32) << 16).view(np.float32)
    return out, lse


@pytest.mark.parametrize("which", ["tiny", "grouped"])
def test_c_program_matches_oracle_and_binding(which, tmp_path):
    if which == "tiny":
        w = named_workload("tiny_bf16")
    else:
        # two units per request, so the launch takes the grouped split
        w = make_workload("c_grouped", seed=91, batch=5, seq_len_range=(2, 1700), num_heads=128, q_len=2,
                          page_size=64, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    out, lse = _run_caller(w, str(tmp_path))
    ref_o, ref_l, rows = oracle_rows(w, list(range(w.batch)))
    check_close(out[rows], ref_o[rows], f"{which} C caller out")
    check_close(lse[rows], ref_l[rows], f"{which} C caller lse")
    # the same library through the Python binding: the same launch, bit for bit
    o2, l2 = run_hip(w, return_lse=True)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
