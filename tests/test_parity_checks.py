"""CPU test: the GPU tests' parity check bites at every output scale.

With the fp8 cache, bmm2 = k_scale = 0.02 (vLLM docs, "FlashInferMLAImpl",
forward_mqa, quantised KV) puts every output far below the bar's absolute
term 1e-2, where |err| <= 1e-2 + 1e-2*|ref| alone would accept an all-zero
result.  gpu_cases.check_close shrinks the absolute term with the outputs and
adds a relative-RMS bound, so that a zeroed, rescaled or noisy result fails
while a correctly rounded (bf16) one passes.  Each case below is the oracle on
the same kind of seeded workload that a GPU test compares against, and the
wrong results are planted here, on the CPU.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_mla_decode_03_amd.inputs import make_workload, INV_SQRT_192, FP8_K_SCALE

from gpu_cases import check_close, ATOL, RTOL


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _fp8_workload(name, seed, **kw):
    base = dict(num_heads=32, q_len=2, page_size=32, kv_dtype="fp8_e4m3fn", kv_value_scale=0.5,
                bmm1_scale=INV_SQRT_192 * FP8_K_SCALE, bmm2_scale=FP8_K_SCALE, causal=True, want_lse=True)
    base.update(kw)
    return make_workload(name, seed=seed, **base)


def _cases():
    """(name, oracle out) pairs in the small-output regimes of the GPU tests."""
    cases = []
    # the device-options tests (sinks, device scales) on the fp8 cache
    w = _fp8_workload("opts", 41, batch=3, seq_len_range=(60, 900))
    cases.append(("options fp8", oracle.reference_decode(oracle.MlaProblem(**w.oracle_problem_kwargs()))[0]))
    # one rank of a sequence-sharded decode on the fp8 cache (rows it sees)
    w = _fp8_workload("dcp", 52, seq_lens=[3, 5, 40, 333, 1200], q_len=3)
    o, l = oracle.reference_dcp_partial(oracle.MlaProblem(**w.oracle_problem_kwargs()), 0, 2)
    cases.append(("dcp rank 0 of 2, fp8", o[~np.isneginf(l)]))
    # a random-sweep case: bmm1 0.02 without the fp8 scale on the cache
    w = make_workload("rand", seed=2003, batch=4, seq_len_range=(1000, 2500), num_heads=48, page_size=16,
                      kv_dtype="fp8_e4m3fn", bmm1_scale=0.02, bmm2_scale=0.5, causal=True, q_len=3)
    cases.append(("random sweep fp8", oracle.reference_decode(oracle.MlaProblem(**w.oracle_problem_kwargs()))[0]))
    # the long-context fp8 workload's settings (H 128, q 2, bmm2 = k_scale) at shorter lengths
    w = _fp8_workload("long", 5, seq_lens=[6000, 9000], num_heads=128, page_size=64)
    cases.append(("long-context fp8", oracle.reference_decode(oracle.MlaProblem(**w.oracle_problem_kwargs()))[0]))
    return cases


@pytest.fixture(scope="module")
def cases():
    return _cases()


def test_the_bare_bar_alone_is_too_weak_here(cases):
    """In these regimes |err| <= 1e-2 + 1e-2*|ref| alone lets almost every
    element be off by 20% (and, for the k_scale outputs, be zero)."""
    for name, ref in cases:
        assert np.mean(np.abs(0.2 * ref) <= ATOL + RTOL * np.abs(ref)) > 0.95, name
        if "fp8" in name and "rank" not in name and "random" not in name:
            assert np.all(np.abs(ref) <= ATOL + RTOL * np.abs(ref)), name


def test_correctly_rounded_results_pass(cases):
    for name, ref in cases:
        check_close(_bf16(ref).astype(np.float32), ref, name)


@pytest.mark.parametrize("plant", ["zeros", "scaled 1.05", "scaled 0.5", "noise 2%", "one head zeroed",
                                   "sign flip"])
def test_planted_wrong_results_fail(cases, plant):
    rng = np.random.default_rng(0)
    for name, ref in cases:
        got = _bf16(ref)
        if plant == "zeros":
            got = np.zeros_like(ref)
        elif plant == "scaled 1.05":
            got = got * 1.05
        elif plant == "scaled 0.5":
            got = got * 0.5
        elif plant == "noise 2%":
            got = got + 0.02 * np.abs(ref).max() * rng.standard_normal(ref.shape)
        elif plant == "one head zeroed":
            got = got.copy()
            got[..., 0, :] = 0.0
        elif plant == "sign flip":
            got = -got
        with pytest.raises(AssertionError):
            check_close(got.astype(np.float32), ref, f"{name} ({plant})")
