"""GPU parity of the fp8-cache path with a bf16 query, where QK^T runs on the
fp8 matrix cores with each (row, head) query split into two E4M3 terms under a
power-of-two scale.  The split is exact for every element within 2^9 of the
pair's largest; the cases here stress what is not: rows whose elements span
many binades, exact zeros, and pairs whose magnitudes sit far from 1 (the scale
exponent at both ends of its range), against the float64 oracle at the usual
bar."""

import numpy as np
import pytest
import torch

from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import make_workload, INV_SQRT_192

from gpu_cases import compare_with_oracle
from helpers import to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_grid():
    binding.set_grid_override(0)
    yield
    binding.set_grid_override(0)


def _bf16_values(bits):
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).float().numpy()


def _workload(name, seed, **kw):
    args = dict(seed=seed, seq_lens=[7, 64, 300, 1999], num_heads=64, q_len=2, page_size=32,
                kv_dtype="fp8_e4m3fn", kv_value_scale=0.5, bmm1_scale=INV_SQRT_192, causal=True, want_lse=True)
    args.update(kw)
    return make_workload(name, **args)


@pytest.mark.parametrize("page_size", [16, 64])
def test_rows_spanning_many_binades(page_size):
    """Elements scaled by 2^u, u uniform in [-24, 3], a tenth of them zero: many
    fall below 2^-9 of their pair's largest, where the low term rounds."""
    w = _workload("split_wide", 90, page_size=page_size)
    rng = np.random.default_rng(91)
    q = _bf16_values(w.q_bits)
    q = q * np.exp2(rng.uniform(-24.0, 3.0, q.shape))
    q[rng.random(q.shape) < 0.1] = 0.0
    w.q_bits = to_bf16_bits(q)
    compare_with_oracle(w)


def test_pair_magnitudes_far_from_one():
    """Whole (row, head) pairs scaled by 2^k, k in {-110, -60, -8, 0, 6, 12}: the
    split's exponent runs from about -6 to 116; the largest pairs give logits
    tens of units past the first tile's maximum (the restart path)."""
    w = _workload("split_scale", 92, bmm1_scale=INV_SQRT_192 / 64.0)
    rng = np.random.default_rng(93)
    q = _bf16_values(w.q_bits)
    ks = np.array([-110, -60, -8, 0, 6, 12], dtype=np.float64)
    q = q * np.exp2(rng.choice(ks, size=q.shape[:2]))[..., None]
    w.q_bits = to_bf16_bits(q)
    compare_with_oracle(w)


def test_zero_rows_and_single_spikes():
    """All-zero pairs (uniform weights) and pairs with one large element among
    tiny ones."""
    w = _workload("split_spike", 94, seq_lens=[2, 33, 512])
    rng = np.random.default_rng(95)
    q = _bf16_values(w.q_bits)
    R, H, D = q.shape
    q[:, ::5] = 0.0
    spikes = rng.random((R, H)) < 0.3
    tiny = q * 2.0 ** -16
    q = np.where(spikes[..., None], tiny, q)
    r, h = np.nonzero(spikes)
    q[r, h, rng.integers(0, D, r.size)] = rng.choice([-6.0, 5.0], r.size)
    w.q_bits = to_bf16_bits(q)
    compare_with_oracle(w)


def test_tiny_scale_with_tiny_pairs():
    """bmm1 = 1e-30 and pairs scaled by 2^-120: the lane's logit scale
    bmm1 log2(e) 2^-e would underflow to zero in float32; it is held at the
    smallest normal float so that every lane of a wave takes the same softmax
    path.  The logits are all ~0: uniform weights, as in the oracle."""
    w = _workload("split_tiny", 96, bmm1_scale=1e-30)
    rng = np.random.default_rng(97)
    q = _bf16_values(w.q_bits)
    q = q * np.exp2(rng.choice(np.array([-120.0, -118.0, 0.0]), size=q.shape[:2]))[..., None]
    w.q_bits = to_bf16_bits(q)
    compare_with_oracle(w)
