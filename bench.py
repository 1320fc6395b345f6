"""Throughput benchmark: batched paged MLA decode on one MI355X.

One step = one mla_decode_paged call (the whole launch: device work plan,
decode and split merge) over the whole batch of a workload, inputs resident
in HBM.  The headline workload is the DeepSeek-V3-shaped bf16 decode (B=64,
H=128, q_len=1, 576/512 dims, seq_lens uniform in [1024, 8192], page size 64,
shuffled pages).

By default every one of the five configured workloads (tiny bf16, the
headline, uniform spec 1+3 causal, ragged packed causal, long-context fp8 KV)
is timed in turn, each with its own warmup and timed steps, the headline
first; the one JSON line carries the headline's figures and, under "configs",
each workload's.  Per workload: KV-tokens/s, TFLOP/s and algorithmic GB/s
over the timed steps, and the roofline fraction of a step (algorithmic bytes
or flops over the device time per step of the timed region, from two HIP
events on the launch stream around it: every kernel of a launch and the gaps
between launches count), plus the decode kernel's own fraction from a
separate pass with events inside each launch.  The float64 CPU oracle is
timed on a bounded sample of the headline workload.

  python bench.py [--gpus 1] [--steps 300] [--warmup 300] [--settle-ms 100]
                  [--workload NAME] [--no-cpu-baseline] [--all]

Before the timed steps of each workload the device runs the warmup steps and
then keeps stepping, untimed, until it has been busy for --settle-ms: after a
load starts, the socket's power controller overshoots for a few tens of
milliseconds (steps run 10-30% slow from about 3 to 40 ms in), and a short
warmup would otherwise put the timed steps inside that transient.  The extra
steps are reported under "settle".

--workload NAME times that workload alone (a paged workload of
paged_mla_decode_03_amd.inputs.WORKLOADS, the fp8-query one of Q8_WORKLOADS or
the sparse top-k one of SPARSE_WORKLOADS); --all adds the fp8-query and sparse
workloads to the default run.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged MLA decode KV-tokens/s and TFLOP/s at 1 GPU; % of MFMA/HBM roofline"
DEFAULT_WORKLOAD = "dsv3_bf16_decode"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, budget_s=10.0, q_codes=None):
    """Time the oracle as it stands on whole requests of w (cycling through the
    batch) until about budget_s seconds of CPU work have been spent (q_codes:
    the fp8 query codes of an fp8-query workload)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    prob = oracle.MlaProblem(**w.oracle_problem_kwargs())
    if q_codes is not None:
        prob.q_bits = q_codes
        prob.q_dtype = "fp8_e4m3fn"
    calls, tokens = 0, 0
    t0 = time.perf_counter()
    while True:
        b = calls % w.batch
        oracle.reference_decode(prob, requests=[b])
        calls += 1
        tokens += int(w.seq_lens[b])
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "KV-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{calls} whole requests of {w.name} (cycling through its {w.batch}), "
                      f"{tokens} KV tokens in {dt:.1f} s, float64 NumPy"}


KERNEL_SRC = os.path.join(ROOT, "paged_mla_decode_03_amd", "csrc", "mla_decode.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_sha256():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def profiled_traffic(workload):
    """HBM bytes per launch (every kernel of one call) from the committed
    rocprofv3 summaries, or None when none matches both the workload and the
    current kernel source.

    A summary carries one line per kernel of the launch
      bench-traffic: workload=W kernel=K kernel_sha256=H fetch_kib=F write_kib=X fetch_scale=a write_scale=b
    where F and X are the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch)
    and a, b the factors that turn them into bytes for a plain copy of known size.
    """
    if not os.path.isdir(PROFILES):
        return None
    sha = kernel_source_sha256()
    total, seen = 0.0, set()
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith((".md", ".txt")):
            continue
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                line = line.strip().strip("`")
                if not line.startswith("bench-traffic:"):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
                key = kv.get("kernel", "decode")
                if kv.get("workload") == workload and kv.get("kernel_sha256") == sha and key not in seen:
                    seen.add(key)
                    total += (float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                              float(kv["write_kib"]) * float(kv["write_scale"])) * 1024
    return int(total) if seen else None


def time_steps(step, steps, warmup, settle_ms=0.0):
    """Run warmup untimed steps, keep stepping (untimed) until the device has
    been busy for settle_ms since the warmup began, then time exactly `steps`
    steps, bracketed by device synchronisation and by two HIP events on the
    launch stream (torch's current stream, which the steps launch on), with
    nothing else inside the region.  The settle period exists because the
    socket's power controller overshoots for a few tens of milliseconds after
    a load starts (steps run 10-30% slow from about 3 to 40 ms in, then settle).
    A second pass of as many steps (at most 500), outside the timed region, has the
    library record events inside every launch, before the decode kernel and
    right after it: those records add a few microseconds to a step, so they
    stay out of the timed one.  Returns (wall ms per step, device ms per step
    over the timed region, mean decode-kernel ms, untimed settle steps)."""
    import numpy as np
    import torch
    from paged_mla_decode_03_amd import binding
    log(f"[bench] warmup {warmup}")
    t_warm = time.perf_counter()
    for _ in range(warmup):
        step()
    settle = 0
    while (time.perf_counter() - t_warm) * 1e3 < settle_ms:
        for _ in range(16):
            step()
        settle += 16
        torch.cuda.synchronize()
    if settle:
        log(f"[bench] settle: {settle} more untimed steps ({settle_ms:.0f} ms of load before timing)")
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} steps")
    t0 = time.perf_counter()
    region[0].record()
    for _ in range(steps):
        step()
    region[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    device_ms = region[0].elapsed_time(region[1]) / steps
    n_ev = min(steps, 500)
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(n_ev)]
    for trio in ev:
        for e in trio:
            e.record()
    torch.cuda.synchronize()
    for i in range(n_ev):
        binding.set_kernel_events(ev[i][0], ev[i][2], ev[i][1])
        step()
    torch.cuda.synchronize()
    binding.set_kernel_events(None, None)
    decode = float(np.mean([a.elapsed_time(b) for a, b, c in ev]))
    return (t1 - t0) * 1e3 / steps, device_ms, decode, settle


def roofline(counts, kern_ms, name, q8=False):
    """A launch (or one kernel of it) timed at kern_ms against its bound: HBM
    if its algorithmic bytes take longer at peak than its algorithmic flops at
    the MFMA peak (bf16; with an fp8 query, QK^T at the fp8 peak and P.V at the
    bf16 one)."""
    from paged_mla_decode_03_amd.metrics import PEAK_HBM_GBS, PEAK_MFMA_TFLOPS, mixed_mfma_peak
    peak_mfma = mixed_mfma_peak() if q8 else PEAK_MFMA_TFLOPS["bf16"]
    t_hbm = counts["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_mfma = counts["flops"] / (peak_mfma * 1e12)
    if t_hbm >= t_mfma:
        achieved = counts["bytes"] / (kern_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": profiled_traffic(name)}
    achieved = counts["flops"] / (kern_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": peak_mfma, "unit": "TFLOP/s",
            "frac": achieved / peak_mfma, "traffic": profiled_traffic(name)}


def sparse_cpu_baseline(w, lists, budget_s=10.0):
    """The sparse oracle as it stands on whole query rows (cycling), about
    budget_s seconds of CPU work."""
    import numpy as np
    from oracle.sparse import reference_sparse_decode
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    R = lists.shape[0]
    calls, tokens = 0, 0
    t0 = time.perf_counter()
    while True:
        r = calls % R
        reference_sparse_decode(w.q_bits[r:r + 1], w.kv_bits, w.kv_dtype, lists[r:r + 1], w.bmm1_scale,
                                w.bmm2_scale)
        calls += 1
        tokens += int((lists[r] >= 0).sum())
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "KV-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{calls} whole query rows of {w.name} (cycling through its {R}), {tokens} listed rows "
                      f"in {dt:.1f} s, float64 NumPy"}


def _result(name, counts, ms_step, device_ms, decode_ms, steps, warmup, dtype, data, config, q8=False,
            settle=None):
    roof = roofline(counts, device_ms, name, q8=q8)
    dec = roofline(counts, decode_ms, name, q8=q8)
    res = {
        "metric": METRIC,
        "value": counts["kv_tokens"] / (ms_step * 1e-3),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": data,
        "config": config,
        "tflops": counts["flops"] / (ms_step * 1e-3) / 1e12,
        "gbps": counts["bytes"] / (ms_step * 1e-3) / 1e9,
        "device_ms_per_step": device_ms,
        "decode_kernel_ms": decode_ms,
        "decode_kernel_frac": dec["frac"],
        "kernel_source_sha256": kernel_source_sha256(),
        "roofline": roof,
    }
    if settle is not None:
        res["settle"] = settle  # the untimed steps run after the warmup (see time_steps)
    return res


def _dtype_label(kv_dtype, q8):
    """The arithmetic each path computes in."""
    if kv_dtype == "bf16":
        return "bf16"
    if q8:
        return "fp8 e4m3 KV and query: QK^T on fp8 MFMA, P.V on bf16 MFMA"
    return ("fp8 e4m3 KV, bf16 query: QK^T on fp8 MFMA (query split into two e4m3 terms), "
            "P.V on bf16 MFMA (V widened exactly)")


def run_sparse_workload(name, steps, warmup, want_cpu, rotate=3, settle_ms=0.0):
    """One step = one sparse top-k decode call over the whole batch."""
    import torch
    from paged_mla_decode_03_amd import binding
    from paged_mla_decode_03_amd.inputs import named_sparse_workload, SPARSE_WORKLOADS
    from paged_mla_decode_03_amd.metrics import sparse_counts

    log(f"[bench] generating workload {name}")
    w, lists = named_sparse_workload(name, poison=False)
    spec = SPARSE_WORKLOADS[name]
    K = int(spec["top_k"])
    counts = sparse_counts(lists, K, w.num_heads, 2 if w.kv_dtype == "bf16" else 1, w.want_lse)
    kv = torch.from_numpy(w.kv_bits)
    kv = (kv.view(torch.bfloat16) if w.kv_dtype == "bf16" else kv.view(torch.float8_e4m3fn)).cuda()
    q = torch.from_numpy(w.q_bits).view(torch.bfloat16).cuda()
    idx = torch.from_numpy(lists).cuda()
    nbytes = binding.sparse_workspace_bytes_for(q, kv, idx, top_k=K, return_lse=w.want_lse)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(tuple(q.shape[:-1]) + (512,), dtype=torch.bfloat16, device="cuda")
    binding.decode_sparse(q, kv, ws, idx, top_k=K, out=out, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale)
    dims, _, _ = binding._sparse_dims(q, kv, idx)
    opts = binding.MlaOptions(None, None, None, None, 1, 0, K)
    stream = torch.cuda.current_stream().cuda_stream
    kvs = [kv] + [kv.clone() for _ in range(max(1, rotate) - 1)]
    qs = [q] + [q.clone() for _ in range(max(1, rotate) - 1)]
    n_step = [0]

    def step():
        i = n_step[0] % len(kvs)
        rc = binding.mla_decode_paged_ex(qs[i].data_ptr(), kvs[i].data_ptr(), idx.data_ptr(), None, None, 1, 1,
                                         w.bmm1_scale, w.bmm2_scale, False, out.data_ptr(), None, ws.data_ptr(),
                                         nbytes, dims, opts, stream=stream)
        n_step[0] += 1
        if rc != 0:
            raise RuntimeError(binding.mla_status_string(rc))

    ms_step, device_ms, decode_ms, settle = time_steps(step, steps, warmup, settle_ms)
    config = {"workload": name, "rows": w.total_q, "heads": w.num_heads, "top_k": K,
              "seq_lens": list(spec["seq_len_range"]), "page_size": w.page_size, "kv_dtype": w.kv_dtype,
              "lse": w.want_lse, "kv_tokens": counts["kv_tokens"]}
    data = (f"synthetic (seeded N(0,1) q/kv, shuffled pages, seeded top-k selections of each request; "
            f"{max(1, rotate)} cache copies rotated across steps)")
    res = _result(name, counts, ms_step, device_ms, decode_ms, steps, warmup,
                  "bf16" if w.kv_dtype == "bf16" else "fp8 e4m3 KV widened exactly to bf16, bf16 MFMA",
                  data, config, settle={"ms": settle_ms, "steps": settle})
    if want_cpu:
        log("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = sparse_cpu_baseline(w, lists)
    return res


def run_workload(name, steps, warmup, want_cpu, rotate=3, settle_ms=0.0):
    import torch
    from paged_mla_decode_03_amd import binding
    from paged_mla_decode_03_amd.inputs import (named_workload, to_device_tensors, WORKLOADS, Q8_WORKLOADS,
                                                fp8_query_codes)
    from paged_mla_decode_03_amd.metrics import counts_for_workload

    log(f"[bench] generating workload {name}")
    q8 = name in Q8_WORKLOADS
    base = Q8_WORKLOADS.get(name, name)
    w = named_workload(base, poison=False)
    counts = counts_for_workload(w)
    t = to_device_tensors(w, "cuda")
    if q8:
        t["q"] = torch.from_numpy(fp8_query_codes(w)).view(torch.float8_e4m3fn).cuda()
    B, H = w.batch, w.num_heads
    q = t["q"] if w.qo_indptr is not None else t["q"].view(B, w.q_len_fixed, H, 576)
    max_q = w.max_q_len if w.qo_indptr is not None else None
    nbytes = binding.workspace_bytes_for(q, t["kv"], t["block_tables"], t["seq_lens"], w.max_seq_len,
                                         qo_indptr=t["qo_indptr"], max_seq_len_q=max_q, return_lse=w.want_lse)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(tuple(q.shape[:-1]) + (512,), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tuple(q.shape[:-1]), dtype=torch.float32, device="cuda") if w.want_lse else None

    # validate once through the checked wrapper, then time the raw C entry point
    binding.decode(q, t["kv"], ws, t["block_tables"], t["seq_lens"], w.max_seq_len, qo_indptr=t["qo_indptr"],
                   max_seq_len_q=max_q, out=out, lse=lse, return_lse=w.want_lse, bmm1_scale=w.bmm1_scale,
                   bmm2_scale=w.bmm2_scale, causal=w.causal)
    dims, max_q_len, _, _ = binding.dims_for(q, t["kv"], t["block_tables"], t["seq_lens"], t["qo_indptr"], max_q)
    stream = torch.cuda.current_stream().cuda_stream
    # Consecutive steps read different copies of the KV cache (and Q), so that a
    # step never finds the previous step's data in L2 or the 256 MB MALL: a
    # serving loop reads each layer's cache once per step.
    kvs = [t["kv"]] + [t["kv"].clone() for _ in range(max(1, rotate) - 1)]
    qs = [q] + [q.clone() for _ in range(max(1, rotate) - 1)]
    arg_sets = [(qq.data_ptr(), kv.data_ptr(), t["block_tables"].data_ptr(), t["seq_lens"].data_ptr(),
                 None if t["qo_indptr"] is None else t["qo_indptr"].data_ptr(), w.max_seq_len, max_q_len,
                 w.bmm1_scale, w.bmm2_scale, w.causal, out.data_ptr(), None if lse is None else lse.data_ptr(),
                 ws.data_ptr(), nbytes, dims) for qq, kv in zip(qs, kvs)]
    opts = binding.MlaOptions(None, None, None, None, 1, 0, 0, 1) if q8 else None
    n_step = [0]

    def step():
        rc = binding.mla_decode_paged_ex(*arg_sets[n_step[0] % len(arg_sets)], opts, stream=stream)
        n_step[0] += 1
        if rc != 0:
            raise RuntimeError(binding.mla_status_string(rc))

    ms_step, device_ms, decode_ms, settle = time_steps(step, steps, warmup, settle_ms)
    spec = WORKLOADS[base]
    config = {"workload": name, "batch": B, "heads": H, **({"q_dtype": "fp8_e4m3fn"} if q8 else {}),
              "q_len": spec.get("q_len") if "q_len_range" not in spec else list(spec["q_len_range"]),
              "seq_lens": list(spec["seq_len_range"]) if "seq_len_range" in spec else
              (list(spec["seq_len_loguniform"]) if "seq_len_loguniform" in spec else spec.get("seq_lens")),
              "page_size": w.page_size, "kv_dtype": w.kv_dtype, "causal": w.causal, "lse": w.want_lse,
              "kv_tokens": counts["kv_tokens"]}
    data = (f"synthetic (seeded N(0,1) q/kv, shuffled pages; {max(1, rotate)} cache copies rotated across steps)"
            + ("; query rounded to fp8 E4M3FN, q_scale 1" if q8 else ""))
    res = _result(name, counts, ms_step, device_ms, decode_ms, steps, warmup, _dtype_label(w.kv_dtype, q8), data,
                  config, q8=q8, settle={"ms": settle_ms, "steps": settle})
    if want_cpu:
        log("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, q_codes=fp8_query_codes(w) if q8 else None)
    return res


def _summary(r):
    """The per-workload figures carried under "configs" of the JSON line."""
    keep = ("value", "unit", "ms_per_step", "device_ms_per_step", "decode_kernel_ms", "decode_kernel_frac", "tflops",
            "gbps", "dtype", "roofline", "settle")
    d = {k: r[k] for k in keep if k in r}
    d["kv_tokens"] = r["config"]["kv_tokens"]
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first: the GPU reaches steady clocks only after tens of ms of work")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="after the warmup steps, keep stepping (untimed, reported as settle.steps) until the "
                         "device has been busy this long: the socket's power controller overshoots for a few "
                         "tens of ms after a load starts; 0 = warmup steps only")
    ap.add_argument("--workload", default=None, help="time this workload alone")
    ap.add_argument("--rotate", type=int, default=3,
                    help="copies of the KV cache and Q read in turn by consecutive steps (1 = one copy, which "
                         "can sit in the 256 MB MALL for the smaller workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="also time the fp8-query and sparse top-k workloads")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed steps, run 3 plain device-to-device copies of this many bytes "
                         "(HBM-counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the decode path is single-GPU by design", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from paged_mla_decode_03_amd.inputs import WORKLOAD_ORDER, SPARSE_WORKLOADS, Q8_WORKLOADS

    def run(name, want_cpu):
        fn = run_sparse_workload if name in SPARSE_WORKLOADS else run_workload
        return fn(name, args.steps, args.warmup, want_cpu, args.rotate, args.settle_ms)

    if args.workload is not None:
        res = run(args.workload, not args.no_cpu_baseline)
        log("[bench] " + json.dumps(_summary(res)))
    else:
        # the five configured workloads, the headline first (the chip warms up
        # over a run of several workloads at the power cap, and later ones read
        # a few per cent slower)
        order = [DEFAULT_WORKLOAD] + [n for n in WORKLOAD_ORDER if n != DEFAULT_WORKLOAD]
        configs = {}
        res = None
        for name in order:
            r = run(name, False)
            configs[name] = _summary(r)
            log(f"[bench] {name}: " + json.dumps(configs[name]))
            if name == DEFAULT_WORKLOAD:
                res = r
        extra = {}
        if args.all:
            for name in list(Q8_WORKLOADS) + list(SPARSE_WORKLOADS):
                extra[name] = _summary(run(name, False))
                log(f"[bench] {name}: " + json.dumps(extra[name]))
        res["configs"] = configs
        if extra:
            res["extra_workloads"] = extra
        if not args.no_cpu_baseline:
            from paged_mla_decode_03_amd.inputs import named_workload
            log("[bench] cpu baseline (oracle)")
            res["cpu_baseline"] = cpu_baseline(named_workload(DEFAULT_WORKLOAD, poison=False))
    if args.copy_bytes > 0:
        n = (args.copy_bytes + 15) // 16 * 16
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copies: 3 x {n} bytes")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
