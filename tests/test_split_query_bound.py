"""The bf16-query split used by the fp8-cache kernels (query mode 2), modelled
on the CPU with torch's own float8 conversion: a (row, head) query q is scaled
by 2^e, e = 8 - frexp_exp(max|q|), and written as q_hi + q_lo, two E4M3 terms.
The kernel's comments and design notes claim that

* the scaled maximum lies in [128, 256) (no E4M3 overflow);
* q_hi + q_lo equals q 2^e exactly for every element with |q 2^e| >= 2^-2,
  i.e. within 2^9 of the pair's largest, for either rounding of q_hi;
* below that the error is at most 2^-10 in scaled units (2^-17 of the largest).

Every finite bf16 value up to the pair's largest is checked, for pair maxima
from 2^-126 to 2^127."""

import numpy as np
import torch


def _e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(
        torch.float32).numpy()


def _all_finite_bf16():
    codes = np.arange(1 << 16, dtype=np.uint32)
    v = (codes << 16).view(np.float32)
    return v[np.isfinite(v)]


def _split(row):
    M = float(np.max(np.abs(row)))
    _, ex = np.frexp(np.float32(M))
    e = 8 - int(ex)
    s = np.ldexp(row.astype(np.float64), e).astype(np.float32)  # exact: a power-of-two scale of bf16 values
    hi = _e4m3(s)
    lo = _e4m3(s - hi)  # s - hi is exact in float32
    return M, e, s, hi, lo


def test_split_is_exact_within_2_pow_9_of_the_largest():
    allv = _all_finite_bf16()
    for M in (2.0 ** -126, 1.5 * 2.0 ** -100, 0.75, 1.0, 3.0, 448.0, 1.5 * 2.0 ** 60, 1.9921875 * 2.0 ** 127):
        row = allv[np.abs(allv) <= M]
        row = np.concatenate([row, [np.float32(M)]])
        Mr, e, s, hi, lo = _split(row)
        assert Mr == M
        sm = float(np.max(np.abs(s)))
        assert 128.0 <= sm < 256.0, (M, sm)
        assert np.all(np.isfinite(hi)) and np.all(np.isfinite(lo))
        err = np.abs(hi.astype(np.float64) + lo.astype(np.float64) - s.astype(np.float64))
        big = np.abs(s) >= 0.25
        assert np.all(err[big] == 0.0), (M, int(np.count_nonzero(err[big])))
        assert np.all(err <= 2.0 ** -10), (M, float(err.max()))
        # relative to the pair's largest: at most 2^-17 (scaled max >= 128)
        assert np.all(err / sm <= 2.0 ** -17)


def test_a_planted_one_term_split_breaks_the_claim():
    """One E4M3 term alone (dropping q_lo) is far from exact: the checks above
    would fail for it, so they do test the second term."""
    allv = _all_finite_bf16()
    row = allv[np.abs(allv) <= 1.0]
    _, _, s, hi, _ = _split(row)
    big = np.abs(s) >= 0.25
    assert np.count_nonzero(hi[big] != s[big]) > 1000
