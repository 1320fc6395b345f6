"""Shared helpers for the GPU parity tests: run the HIP path on a seeded
workload and compare with the float64 oracle on the same inputs."""

import numpy as np
import torch

import oracle
from paged_mla_decode_03_amd import binding
from paged_mla_decode_03_amd.inputs import to_device_tensors

ATOL = 1e-2
RTOL = 1e-2
# Bug signals that hold at any output scale (bf16 outputs carry about 2^-9
# relative rounding, and the path adds a few such roundings at most).
REL_RMS_LIMIT = 5e-3
REL_MAX_LIMIT = 1e-2


def run_hip(w, *, return_lse=None, out=None, kv_rank4=False, stream=None):
    """Run the library on workload w.  Returns (out float32 [R, H, 512], lse float32 [R, H] or None)."""
    t = to_device_tensors(w, "cuda")
    B, H = w.batch, w.num_heads
    q = t["q"]
    if w.qo_indptr is None:
        q = q.view(B, w.q_len_fixed, H, 576)
    kv = t["kv"]
    if kv_rank4:
        kv = kv.unsqueeze(1)
    want_lse = w.want_lse if return_lse is None else return_lse
    nbytes = binding.workspace_bytes_for(q, kv, t["block_tables"], t["seq_lens"], w.max_seq_len,
                                         qo_indptr=t["qo_indptr"], max_seq_len_q=w.max_q_len,
                                         return_lse=want_lse)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    res = binding.decode(q, kv, ws, t["block_tables"], t["seq_lens"], w.max_seq_len, qo_indptr=t["qo_indptr"],
                         max_seq_len_q=w.max_q_len if w.qo_indptr is not None else None, out=out,
                         return_lse=want_lse, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale, causal=w.causal)
    torch.cuda.synchronize()
    o, l = res if want_lse else (res, None)
    o = o.float().reshape(w.total_q, H, 512).cpu().numpy()
    l = None if l is None else l.reshape(w.total_q, H).cpu().numpy()
    return o, l


def oracle_rows(w, requests):
    prob = oracle.MlaProblem(**w.oracle_problem_kwargs())
    out, lse = oracle.reference_decode(prob, requests=requests)
    rows = []
    for b in requests:
        r0, qb = prob.request_rows(b)
        rows.extend(range(r0, r0 + qb))
    return out, lse, np.array(rows, dtype=np.int64)


def check_close(got, ref, what, atol=ATOL, rtol=RTOL, rel_rms_limit=REL_RMS_LIMIT, rel_max_limit=REL_MAX_LIMIT):
    """The parity bar, made scale-aware so that it bites at every output scale.

    * elementwise |got - ref| <= a + rtol*|ref| with a = min(atol, rel_max_limit * max|ref|):
      the stated bar |err| <= 1e-2 + 1e-2*|ref| where outputs are O(1), and no
      looser than it anywhere; where every |ref| is far below 1e-2 (fp8 caches
      with bmm2 = k_scale) the absolute term shrinks with the outputs, so an
      all-zero or badly scaled result fails;
    * relative RMS error sqrt(mean err^2) / sqrt(mean ref^2) < rel_rms_limit.
    Returns (relative RMS, max |err|)."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got.astype(np.float64) - ref)
    ref_max = float(np.abs(ref).max()) if ref.size else 0.0
    a = min(atol, rel_max_limit * ref_max)
    bound = a + rtol * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance "
                           f"(absolute term {a:.3e}); max err {err.max():.3e} at "
                           f"{np.unravel_index(err.argmax(), err.shape)}")
    ref_rms = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    rms = float(np.sqrt((err ** 2).mean())) / ref_rms if ref_rms > 0 else (0.0 if not err.any() else np.inf)
    assert rms < rel_rms_limit, f"{what}: relative RMS error {rms:.2e} above {rel_rms_limit:.0e}"
    return float(rms), float(err.max()) if err.size else 0.0


def compare_with_oracle(w, requests=None, **run_kw):
    if requests is None:
        requests = list(range(w.batch))
    got_o, got_l = run_hip(w, **run_kw)
    ref_o, ref_l, rows = oracle_rows(w, requests)
    rms, mx = check_close(got_o[rows], ref_o[rows], f"{w.name} out")
    stats = {"out_rel_rms": rms, "out_max_err": mx}
    if got_l is not None:
        lrms, lmx = check_close(got_l[rows], ref_l[rows], f"{w.name} lse")
        stats.update(lse_rel_rms=lrms, lse_max_err=lmx)
    return stats

