"""Benchmark of the fused Global-QSGD compress + integer sum + dequantize path.

One step = one gq_compress_mean call over one batch of n simulated workers'
gradient shards already resident in HBM: the global (q,p)-norm pass, then
the fused quantize / exact integer sum / dequantize pass.  The default
workload is the largest fp32 one that fits one GPU: n = 64 workers x
d = 64,000,000 fp32 coordinates (16.4 GB), standard dithering, s = 3,
q = p = 2, with local-norm QSGD timed beside it.  The three other large
workloads (ResNet-50-, BERT-base- and GPT-2-medium-sized buckets) are timed
in the same run and reported under "configs".

Prints one JSON line.  `value` is input GB/s (n d bytes-per-element / step
time); `roofline` describes the dominant kernel (pass 1, which reads x
whole: k_norm_oneshot or k_norm_partial) timed per launch with HIP events on
the stream it runs on, and `compress_step` the fused pass with the zero-code
skip (bound by the vector ALU: Philox for every worker and group) beside the
same pass reading every coordinate; `read_ceiling` is the best
plain stream read of the same input (libgq_probe.so), `valu_ceiling` the
measured issue rate of the instruction kinds the VALU-heavy kernels use;
`e8_omega` the byte rate of the pages' 8-bit custom reduction against an
fp32 sum; `cpu_baseline` is the CPU oracle on every host core (and on one)
over a bounded prefix of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, help="workload key in workloads.WORKLOADS")
    ap.add_argument("--configs", default="2,3,4",
                    help="other workload keys timed in the same run ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the multi-threaded oracle baseline (0 disables it)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the read ceiling, VALU rates, 8-bit omega and DDP hook figures "
                         "(counter passes of one workload)")
    ap.add_argument("--valu-probe", action="store_true",
                    help="with --no-extras: still run the VALU issue-rate probe kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--unfused", action="store_true", help="also time the four-call unfused path")
    ap.add_argument("--words", action="store_true",
                    help="also time the word layout for a native uint32 SUM all-reduce")
    ap.add_argument("--bucket", action="store_true",
                    help="also time one device's share of a data-parallel gradient bucket "
                         "(1, 25 and 100 MB of worker 0's row)")
    ap.add_argument("--e8", action="store_true",
                    help="also measure the 8-bit exponential format: its pair reduction against "
                         "fp32/uint8 sums (omega) and the fused tree path on this workload")
    ap.add_argument("--ablation", action="store_true",
                    help="also time local-norm QSGD on the same input (default on workload 5)")
    return ap.parse_args()


def source_hash() -> str:
    """Hash of the kernel source with // comments, indentation and line
    breaks removed, so that only code changes invalidate a stored counter
    record."""
    with open(os.path.join(ROOT, "allreduce_compatible_gradient_amd", "csrc", "gq.hip")) as f:
        code = "".join(line.split("//", 1)[0].strip() for line in f)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_for(workload_name: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload_name)
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def event_pairs(torch, k):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(k)]


def cpu_baseline(w, target_s: float):
    """The oracle as it is (scalar C, never tuned for this) on the first d'
    coordinates of every worker: the whole operation (norm, codes, exact
    sum, dequantization).  On every host core the rows' norms and then
    blocks of columns run in a pool of threads, each block one oracle call;
    the one-core figure is one oracle call over a smaller prefix."""
    import oracle
    import workloads as wl
    scheme = oracle.SCHEME_L if w.scheme == "L" else oracle.SCHEME_E
    threads = oracle._threads(None)
    d0 = min(w.d, 1 << 15)
    x = wl.generate(w, d=d0)
    t0 = time.perf_counter()
    oracle.compress_mean(x, w.s, w.q, w.p, scheme, w.seed)
    per_elem = (time.perf_counter() - t0) / (w.n * d0)   # one core, seconds per element

    def whole(xs, nthreads):
        t0 = time.perf_counter()
        N, _ = oracle.global_norm_rows(xs, w.q, w.p, threads=nthreads)
        oracle.compress_mean_all(xs, N, w.s, scheme, w.seed, threads=nthreads)
        return time.perf_counter() - t0

    # all host threads: about target_s of wall time
    d1 = int(min(w.d, max(d0, target_s * threads / per_elem / w.n)))
    x = wl.generate(w, d=d1, threads=threads)
    dt = whole(x, threads)
    del x
    # one thread: a third of that time
    d2 = int(min(w.d, max(d0, target_s / 3.0 / per_elem / w.n)))
    x = wl.generate(w, d=d2, threads=threads)
    t0 = time.perf_counter()
    oracle.compress_mean(x, w.s, w.q, w.p, scheme, w.seed)
    dt1 = time.perf_counter() - t0
    del x
    gbs = w.n * d1 * w.elem_bytes / dt / 1e9
    gbs1 = w.n * d2 * w.elem_bytes / dt1 / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {d1} of {w.d} coordinates of all {w.n} workers "
                      f"({w.n * d1} elements, {dt:.1f} s on {threads} threads: row norms, then "
                      f"column blocks, each block one oracle call)",
            "cpu_model": _cpu_model(),
            "one_core": {"value": round(gbs1, 6), "unit": "GB/s", "cores": 1,
                         "sample": f"first {d2} coordinates of all {w.n} workers "
                                   f"({w.n * d2} elements, {dt1:.1f} s, one oracle call)"}}


def _cpu_model() -> str:
    """The host CPU's model name (Linux), for the CPU baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def eq8_threshold(rho: float, omega: float) -> float:
    """Largest beta / gamma at which the compressed Allreduce is faster.

    Reading of Eq. (8) of "Global-QSGD: Practical Floatless Quantization ..."
    (Sec. 5 performance model, delta = 0): with rho = S / S_hat and omega =
    gamma_hat / gamma (byte rates of the custom and the fp32 reduction),
    compression pays iff (1/gamma)(1/(rho omega) - 1) < (2/beta)(1 - 1/rho).
    Returns inf when it always pays (rho omega >= 1)."""
    lhs = 1.0 / (rho * omega) - 1.0
    return math.inf if lhs <= 0 else 2.0 * (1.0 - 1.0 / rho) / lhs


def _time_us(torch, stream, fn, reps):
    """Device time per call of fn(stream), in microseconds.  The reps calls
    are captured in one HIP graph and replayed, so that calls shorter than
    the host's per-call overhead are still timed back to back on the GPU."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _ in range(3):
            fn(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(reps):
            fn(side)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / reps * 1e3


def e8_omega(gq, torch, stream, dev):
    """omega of the pages' 8-bit custom reduction ("Global-QSGD: Practical
    Floatless Quantization ...", Sec. 5: the byte rate of the custom pair
    reduction over that of an fp32 sum), with omega_S of a plain uint8 sum,
    at the pages' 25 MB bucket and at 1 GB."""
    out = {}
    g = torch.Generator(device="cpu").manual_seed(0)
    for label, nbytes in (("25MB", 25 << 20), ("1GB", 1 << 30)):
        d = nbytes // 4  # elements of an fp32 buffer of that size
        a = torch.randn(d, generator=g).to(dev)
        b = torch.randn(d, generator=g).to(dev)
        c = torch.empty_like(a)
        t_f32 = _time_us(torch, stream, lambda st: torch.add(a, b, out=c), 50)
        au = torch.randint(0, 256, (d,), dtype=torch.uint8, generator=g).to(dev)
        bu = torch.randint(0, 256, (d,), dtype=torch.uint8, generator=g).to(dev)
        cu = torch.empty_like(au)
        t_u8 = _time_us(torch, stream, lambda st: torch.add(au, bu, out=cu), 50)
        t_e8 = _time_us(torch, stream, lambda st: gq.gq_e8_reduce_pair(au, bu, d, 1, 1, 0, out=cu,
                                                                       stream=st), 50)
        del a, b, c
        # byte rates: the fp32 sum reduces 4d bytes, the code sums d bytes
        om_e, om_s = (d / t_e8) / (4 * d / t_f32), (d / t_u8) / (4 * d / t_f32)
        out[label] = {"elements": d, "fp32_sum_us": round(t_f32, 3), "u8_sum_us": round(t_u8, 3),
                      "e8_pair_reduce_us": round(t_e8, 3), "omega_E": round(om_e, 4),
                      "omega_S": round(om_s, 4),
                      "eq8_beta_over_gamma_E": eq8_threshold(4.0, om_e)}
        del au, bu, cu
    torch.cuda.empty_cache()
    return out


def e8_report(gq, torch, w, xd, stream, steps, ws):
    """The 8-bit exponential format: omega of its custom pair reduction, and
    the fused norm + codes + re-rounding tree + dequantization path."""
    out = e8_omega(gq, torch, stream, xd.device)
    n, d = w.n, w.d
    if n & (n - 1) == 0:
        mean = torch.empty(d, dtype=torch.float32, device=xd.device)
        norm = torch.empty(1, dtype=torch.float32, device=xd.device)
        t = _time_us(torch, stream, lambda st: gq.gq_e8_compress_mean(
            xd, w.q, w.p, w.seed, mean=mean, norm=norm, workspace=ws, stream=st), steps)
        out["fused"] = {"ms_per_step": round(t * 1e-3, 6),
                        "input_GBs": round(n * d * w.elem_bytes / (t * 1e-6) / 1e9, 3),
                        "bits_per_element": 8}
        # the same steps as separate calls: codes of every worker, the tree
        # over the stored codes, dequantization of the root
        codes = torch.empty((n, gq.gq_e8_row_bytes(d)), dtype=torch.uint8, device=xd.device)
        root = torch.empty(gq.gq_e8_row_bytes(d), dtype=torch.uint8, device=xd.device)
        gq.gq_global_norm(xd, w.q, w.p, norm=norm, workspace=ws, stream=stream)
        parts = {
            "e8_quantize_us": lambda st: gq.gq_e8_quantize(xd, norm, w.seed, codes=codes,
                                                           stream=st),
            "e8_tree_us": lambda st: gq.gq_e8_tree(codes, n, d, w.seed, root=root, stream=st),
            "e8_dequantize_us": lambda st: gq.gq_e8_dequantize(root, d, norm, mean=mean,
                                                               stream=st),
        }
        out["unfused"] = {k: round(_time_us(torch, stream, f, steps), 3) for k, f in parts.items()}
        del codes, root
    return out


def bucket_report(gq, torch, w, xd, stream, steps):
    """One device's share of a data-parallel gradient bucket, device 0 of
    n = w.n workers: the fp64 norm term of its bucket, N from the term (after
    what would be an all-reduce of that double), its codes at its worker
    index in the word layout of the width that holds a sum of n codes (what
    a native uint32 SUM all-reduce adds), and the mean from the summed words
    (after what would be that all-reduce; here the device's own row stands
    in for the sum).  The two all-reduces are not run: the library works on
    one device.  Buckets are the leading 1, 25 and 100 MB of worker 0's row, timed
    as graph replays of the four launches; "with_skip" times the same share
    with the term-and-bounds pass and the zero-code skip in place of the
    first and third launches."""
    out = {}
    W = gq.gq_min_code_bits(w.n, w.s, w.scheme)
    for label, nbytes in (("1MB", 1 << 20), ("25MB", 25 << 20), ("100MB", 100 << 20)):
        db = min(nbytes // w.elem_bytes, w.d)
        b = xd[0, :db].clone().view(1, db)
        ws = torch.empty(gq.gq_workspace_bytes(1, db), dtype=torch.uint8, device=xd.device)
        term = torch.empty(1, dtype=torch.float64, device=xd.device)
        norm = torch.empty(1, dtype=torch.float32, device=xd.device)
        rb = gq.gq_word_row_bytes(db, W)
        words = torch.empty((1, rb // 4), dtype=torch.int32, device=xd.device)
        mean = torch.empty(db, dtype=torch.float32, device=xd.device)
        bounds = torch.empty(gq.gq_span_bounds_bytes(1, db), dtype=torch.uint8, device=xd.device)
        parts = {
            "norm_term_us": lambda st: gq.gq_norm_term(b, w.q, w.p, term=term, workspace=ws,
                                                       stream=st),
            "norm_from_term_us": lambda st: gq.gq_norm_from_term(term, w.q, w.p, norm=norm,
                                                                 stream=st),
            "quantize_words_us": lambda st: gq.gq_quantize_words(b, w.s, w.scheme, norm, w.seed,
                                                                 W, worker_base=0, words=words,
                                                                 stream=st),
            "dequantize_words_us": lambda st: gq.gq_dequantize_words(words[0], w.n, db, w.s,
                                                                     w.scheme, W, norm,
                                                                     mean=mean, stream=st),
        }

        skip_parts = {
            "norm_term_bounds_us": lambda st: gq.gq_norm_term_bounds(
                b, w.q, w.p, term=term, bounds=bounds, workspace=ws, stream=st),
            "norm_from_term_us": parts["norm_from_term_us"],
            "compress_words_skip_us": lambda st: gq.gq_compress_words_skip(
                b, w.s, w.scheme, norm, bounds, w.seed, W, word_sum=words[0], stream=st),
            "dequantize_words_us": parts["dequantize_words_us"],
        }

        def share(st):
            for f in parts.values():
                f(st)

        def share_skip(st):
            for f in skip_parts.values():
                f(st)
        t = _time_us(torch, stream, share, steps)
        t_skip = _time_us(torch, stream, share_skip, steps)
        # algorithmic bytes: the bucket read twice, the word row written and read, the mean
        alg = 2 * db * w.elem_bytes + 2 * rb + 4 * db
        out[label] = {"elements": db, "code_bits": W, "us": round(t, 3),
                      "bucket_GBs": round(db * w.elem_bytes / (t * 1e-6) / 1e9, 3),
                      "alg_GBs": round(alg / (t * 1e-6) / 1e9, 3),
                      "wire_bytes": rb, "bits_on_wire": round(8.0 * rb / db, 3),
                      **{k: round(_time_us(torch, stream, f, steps), 3) for k, f in parts.items()},
                      "with_skip": {
                          "us": round(t_skip, 3),
                          **{k: round(_time_us(torch, stream, skip_parts[k], steps), 3)
                             for k in ("norm_term_bounds_us", "compress_words_skip_us")}}}
        del b, ws, words, mean, bounds
    return out


def words_report(gq, torch, w, xd, stream, steps, norm, mean):
    """The word layout at the minimal width: floor(32 / W) biased fields per
    32-bit word, so that a native uint32 SUM all-reduce adds the codes.
    Times the codes of all n rows, the word-wise sum over the rows (the
    all-reduce's arithmetic, on one device), the same summed row in one pass
    (what a device holding the n rows sends) reading every coordinate and
    with the zero-code skip (given the term-and-bounds pass, timed too), and
    the dequantization, with bits on the wire per coordinate against an int32
    container.  The skipped row is checked equal to the dense one."""
    n, d = w.n, w.d
    W = gq.gq_min_code_bits(n, w.s, w.scheme)
    rb = gq.gq_word_row_bytes(d, W)
    words = torch.empty((n, rb // 4), dtype=torch.int32, device=xd.device)
    wsum = torch.empty(rb // 4, dtype=torch.int32, device=xd.device)
    wskip = torch.empty(rb // 4, dtype=torch.int32, device=xd.device)
    term = torch.empty(1, dtype=torch.float64, device=xd.device)
    bounds = torch.empty(gq.gq_span_bounds_bytes(n, d), dtype=torch.uint8, device=xd.device)
    ws = torch.empty(gq.gq_workspace_bytes(n, d), dtype=torch.uint8, device=xd.device)
    gq.gq_norm_term_bounds(xd, w.q, w.p, term=term, bounds=bounds, workspace=ws, stream=stream)
    parts = {
        "quantize_words_us": lambda st: gq.gq_quantize_words(xd, w.s, w.scheme, norm, w.seed, W,
                                                             words=words, stream=st),
        "sum_words_us": lambda st: gq.gq_sum_words(words, n, d, W, word_sum=wsum, stream=st),
        "compress_words_us": lambda st: gq.gq_compress_words_from_norm(
            xd, w.s, w.scheme, norm, w.seed, W, word_sum=wsum, stream=st),
        "norm_term_bounds_us": lambda st: gq.gq_norm_term_bounds(
            xd, w.q, w.p, term=term, bounds=bounds, workspace=ws, stream=st),
        "compress_words_skip_us": lambda st: gq.gq_compress_words_skip(
            xd, w.s, w.scheme, norm, bounds, w.seed, W, word_sum=wskip, stream=st),
        "dequantize_words_us": lambda st: gq.gq_dequantize_words(wsum, n, d, w.s, w.scheme, W,
                                                                 norm, mean=mean, stream=st),
    }
    out = {"code_bits": W, "fields_per_word": 32 // W, "bits_on_wire": 8.0 * rb / d,
           "row_bytes": rb}
    in_bytes = n * d * w.elem_bytes
    # the skip's rate is still quoted over the input it stands for
    alg = {"quantize_words_us": in_bytes + n * rb, "sum_words_us": (n + 1) * rb,
           "compress_words_us": in_bytes + rb,
           "norm_term_bounds_us": in_bytes + gq.gq_span_bounds_bytes(n, d),
           "compress_words_skip_us": in_bytes + rb,
           "dequantize_words_us": rb + 4 * d}
    for k, f in parts.items():
        t = _time_us(torch, stream, f, steps)
        out[k] = round(t, 3)
        out[k.replace("_us", "_alg_GBs")] = round(alg[k] / (t * 1e-6) / 1e9, 1)
    torch.cuda.synchronize()
    out["skip_row_equals_dense"] = bool(torch.equal(wskip, wsum))
    out["device_step_us"] = {
        "reading_every_coordinate": round(out["norm_term_bounds_us"] + out["compress_words_us"], 3),
        "with_the_skip": round(out["norm_term_bounds_us"] + out["compress_words_skip_us"], 3)}
    del words, wsum, wskip, bounds, ws
    return out


def ablation(gq, torch, w, xd, stream, steps, global_ms, gmean, gnorm, ws):
    """Global-L_s against per-worker local-norm QSGD on the same input: time,
    bits sent per element, and the relative error of the dequantized mean."""
    n, d = w.n, w.d
    lmean = torch.empty(d, dtype=torch.float32, device=xd.device)
    norms = torch.empty(n, dtype=torch.float32, device=xd.device)

    def lstep():
        gq.gq_qsgd_local_mean(xd, w.s, w.seed, mean=lmean, norms=norms, workspace=ws,
                              stream=stream)
    for _ in range(3):
        lstep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        lstep()
    e1.record(stream)
    torch.cuda.synchronize()
    lms = e0.elapsed_time(e1) / steps
    # accuracy against the exact mean (fp64 reference; a reporting aid, not the path)
    gq.gq_compress_mean(xd, w.s, w.q, w.p, w.scheme, w.seed, mean=gmean, norm=gnorm,
                        workspace=ws, stream=stream)
    torch.cuda.synchronize()
    ref = torch.zeros(d, dtype=torch.float64, device=xd.device)
    for i in range(n):
        ref += xd[i].double()
    ref /= n
    den = float((ref * ref).sum())

    def rel(m):
        return float(((m.double() - ref) ** 2).sum()) / den
    in_bytes = n * d * w.elem_bytes
    wl_bits = gq.gq_min_code_bits(1, w.s, "L")  # per-worker local codes: [-s, s]
    return {
        "global": {"ms_per_step": round(global_ms, 6),
                   "input_GBs": round(in_bytes / (global_ms * 1e-3) / 1e9, 3),
                   "code_bits": w.code_bits, "bits_per_element": w.code_bits,
                   "rel_sq_error_of_mean": rel(gmean), "allreduce_compatible": True},
        "local_qsgd": {"ms_per_step": round(lms, 6),
                       "input_GBs": round(in_bytes / (lms * 1e-3) / 1e9, 3),
                       "code_bits": wl_bits, "bits_per_element": wl_bits + 32.0 / d,
                       "rel_sq_error_of_mean": rel(lmean), "allreduce_compatible": False},
    }


def load_workload(np, torch, wl, w, dev):
    """Generate workload w on the host (seeded, threads) and copy it to the device."""
    t0 = time.perf_counter()
    x = wl.generate(w, threads=min(16, os.cpu_count() or 1))
    xd = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(dev)
    if w.dtype == "bf16":
        xd = xd.view(torch.bfloat16)
    del x
    return xd, time.perf_counter() - t0


def workload_config(w, wmin):
    return {"workload": w.name, "scheme": f"Global-{w.scheme}_s", "s": w.s,
            "q": w.q if w.q != float("inf") else "inf",
            "p": w.p if w.p != float("inf") else "inf",
            "n_workers": w.n, "d": w.d, "input_dtype": w.dtype, "code_bits": w.code_bits,
            "min_code_bits": wmin, "values": w.values}


def norm_pass_kernel(w):
    """The kernel that reads x in pass 1: one-shot 16 KB blocks for inputs
    above 256 MiB, chunk-major blocks otherwise."""
    big = w.n * w.d * w.elem_bytes > (1 << 28)
    return "k_norm_oneshot" if big else "k_norm_partial"


# Vector ALU issue ceiling (wave64 VOP3 instructions per CU per clock, probe
# kernels in libgq_probe.so) times 256 CUs x 64 lanes x 2.4 GHz
VALU_LANE_OPS = 0.969 * 256 * 64 * 2.4e9


def skip_alu_roofline(w, k_ms):
    """The fused pass with the zero-code skip is bound by the vector ALU: every
    (worker, 8-coordinate group) needs its Philox4x32-10 block whether or not
    its codes are 0.  Algorithmic work: 40 lane-instructions per block (10
    rounds of two 32x32->64 products and two three-input xors) against the
    measured issue ceiling."""
    blocks = w.n * -(-w.d // 8)
    achieved = 40 * blocks / (k_ms * 1e-3)
    return {"bound": "alu", "achieved": round(achieved / 1e12, 3), "peak": round(VALU_LANE_OPS / 1e12, 3),
            "unit": "T lane-instr/s (Philox only)", "frac": round(achieved / VALU_LANE_OPS, 4),
            "kernel": "k_compress_mean (zero-code skip)"}


def time_workload(gq, np, torch, w, xd, stream, steps, warmup, full):
    """The whole step (norm pass + fused pass) over `steps` back-to-back calls,
    then each pass alone with one HIP event pair per launch on the stream it
    runs on.  full: also cold-cache and graph-replayed step times."""
    n, d = w.n, w.d
    dev = xd.device
    mean = torch.empty(d, dtype=torch.float32, device=dev)
    norm = torch.empty(1, dtype=torch.float32, device=dev)
    # the workspace with which gq_compress_mean is fastest (room for the span
    # bounds of the zero-code skip)
    ws = torch.empty(gq.gq_compress_workspace_bytes(n, d), dtype=torch.uint8, device=dev)

    def step():
        gq.gq_compress_mean(xd, w.s, w.q, w.p, w.scheme, w.seed, mean=mean, norm=norm,
                            workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    in_bytes = n * d * w.elem_bytes
    out = {}
    if full:
        # the same step with the caches cold: reading 1 GiB before each step
        # evicts L2 and the 256 MB Infinity Cache, so no step re-reads what
        # the previous one left there.  The flush only reads, so it leaves no
        # dirty lines to be written back inside the step.
        flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        fsum = torch.empty((), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        cpairs = event_pairs(torch, min(steps, 20))
        for a, b in cpairs:
            torch.sum(flush, 0, out=fsum)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        cold_ms = float(np.median([a.elapsed_time(b) for a, b in cpairs]))
        del flush
        # graph replays: device time without host launch overhead (what bounds
        # the small workload is the launches themselves)
        graph_us = _time_us(torch, stream, lambda st: gq.gq_compress_mean(
            xd, w.s, w.q, w.p, w.scheme, w.seed, mean=mean, norm=norm, workspace=ws, stream=st),
            min(steps, 50))
        out["graph_replay"] = {"ms_per_step": round(graph_us * 1e-3, 6),
                               "input_GBs": round(in_bytes / (graph_us * 1e-6) / 1e9, 3)}
        out["cold_cache"] = {"ms_per_step": round(cold_ms, 6),
                             "input_GBs": round(in_bytes / (cold_ms * 1e-3) / 1e9, 3),
                             "steps": len(cpairs), "stat": "median"}
    # each pass of the step alone, one event pair per launch on the stream it
    # runs on: pass 1 (the norm, and the span bounds in the same read) and the
    # fused pass with the zero-code skip -- the two halves gq_compress_mean
    # runs with this workspace -- and, for comparison, the fused pass reading
    # every coordinate (gq_compress_mean_from_norm)
    bounds = torch.empty(gq.gq_span_bounds_bytes(n, d), dtype=torch.uint8, device=dev)
    npairs, kpairs = event_pairs(torch, steps), event_pairs(torch, steps)
    for i in range(steps):
        npairs[i][0].record(stream)
        gq.gq_global_norm_bounds(xd, w.q, w.p, norm=norm, bounds=bounds, workspace=ws,
                                 stream=stream)
        npairs[i][1].record(stream)
        kpairs[i][0].record(stream)
        gq.gq_compress_mean_skip(xd, w.s, w.scheme, w.seed, norm, bounds, mean=mean,
                                 stream=stream)
        kpairs[i][1].record(stream)
    dpairs = event_pairs(torch, min(steps, 10))
    dense_mean = torch.empty_like(mean)
    for a, b in dpairs:
        a.record(stream)
        gq.gq_compress_mean_from_norm(xd, w.s, w.scheme, w.seed, norm, mean=dense_mean,
                                      stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    if not torch.equal(dense_mean.view(torch.int32), mean.view(torch.int32)):
        raise RuntimeError("the fused pass with and without the zero-code skip disagree")
    del dense_mean
    n_ms = float(np.mean([a.elapsed_time(b) for a, b in npairs]))
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in kpairs]))
    dense_ms = float(np.mean([a.elapsed_time(b) for a, b in dpairs]))
    norm_kernel = norm_pass_kernel(w)
    # pass 1 is the dominant kernel: algorithmic bytes = one read of x and the
    # span bounds it writes
    b_bytes = gq.gq_span_bounds_bytes(n, d)
    n_alg = in_bytes + b_bytes
    fused_alg = 2 * in_bytes + 4 * d              # both passes of the whole step (8d)
    traffic = traffic_for(w.name)
    if n_ms >= k_ms:
        achieved = n_alg / (n_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "kernel": norm_kernel, "alg_bytes_per_launch": n_alg,
                    "traffic_over_alg": round(traffic / n_alg, 4) if traffic else None}
    else:
        roofline = skip_alu_roofline(w, k_ms)
    out.update({
        "ms_per_step": round(ms, 6),
        "input_GBs": round(in_bytes / (ms * 1e-3) / 1e9, 3),
        # the 8d roofline fraction: two reads of x and the fp32 mean over the
        # step time; the skip re-reads only the groups that may hold a
        # non-zero code, so this counts bytes the step no longer moves
        "hbm_frac_fused": round(fused_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_ms": {"norm_pass": round(n_ms, 6), "k_compress_mean (zero-code skip)":
                       round(k_ms, 6)},
        "compress_step": {"ms": round(k_ms, 6), "ms_reading_every_coordinate": round(dense_ms, 6),
                          "speedup_of_skip": round(dense_ms / k_ms, 3),
                          "alu": skip_alu_roofline(w, k_ms)},
        "roofline": roofline,
        "_mean": mean, "_norm": norm, "_ws": ws,
    })
    return out


class _Bucket:
    """The part of DDP's GradBucket the hook reads: a flat gradient buffer and its index."""

    def __init__(self, buf, index):
        self._buf, self._index = buf, index

    def buffer(self):
        return self._buf

    def index(self):
        return self._index


def _hook_device_us(torch, stream, state, buf, steps):
    """Device time of the hook's four library launches for one bucket (norm
    term, N from the term, codes in the word layout, dequantization), with
    the two collectives left out: graph replays, so host time is excluded."""
    import allreduce_compatible_gradient_amd as gq
    d = buf.numel()
    W = gq.gq_min_code_bits(1, state.s, state.scheme)
    x = buf.view(1, -1)
    term = torch.empty(1, dtype=torch.float64, device=buf.device)
    norm = torch.empty(1, dtype=torch.float32, device=buf.device)
    ws = torch.empty(max(gq.gq_workspace_bytes(1, d), 16), dtype=torch.uint8, device=buf.device)
    words = torch.empty((1, gq.gq_word_row_bytes(d, W) // 4), dtype=torch.int32, device=buf.device)
    mean = torch.empty(d, dtype=torch.float32, device=buf.device)

    def launches(st):
        gq.gq_norm_term(x, state.q, state.p, term=term, workspace=ws, stream=st)
        gq.gq_norm_from_term(term, state.q, state.p, norm=norm, stream=st)
        gq.gq_quantize_words(x, state.s, state.scheme, norm, state.seed, W, words=words, stream=st)
        gq.gq_dequantize_words(words[0], 1, d, state.s, state.scheme, W, norm, mean=mean, stream=st)
    return _time_us(torch, stream, launches, steps)


def ddp_hook_report(torch, w, stream, steps):
    """The DDP communication hook (allreduce_compatible_gradient_amd.ddp) on one
    rank over RCCL, per gradient bucket of 25 and 100 MB: the norm term, its
    all-reduce, N, the codes in the word layout, the integer all-reduce and
    the dequantization, with the workload's scheme and orders.  `us` is the
    wall time per bucket of back-to-back hook calls (host work included, as
    DDP would see it), `latency_us` that of one call waited for alone, and
    `device_us` the GPU time of the hook's four library launches."""
    import socket

    import torch.distributed as dist

    from allreduce_compatible_gradient_amd.ddp import GlobalQSGDState, global_qsgd_hook
    with socket.socket() as sk:
        sk.bind(("127.0.0.1", 0))
        port = sk.getsockname()[1]
    dist.init_process_group("nccl", init_method=f"tcp://127.0.0.1:{port}", rank=0, world_size=1)
    out = {"scheme": f"Global-{w.scheme}_s", "s": w.s, "world": 1}
    try:
        state = GlobalQSGDState(scheme=w.scheme, s=w.s, q=w.q, p=w.p, seed=w.seed)
        g = torch.Generator(device="cuda").manual_seed(0)
        for label, nbytes in (("25MB", 25 << 20), ("100MB", 100 << 20)):
            buf = torch.randn(nbytes // 4, device="cuda", generator=g) * 1e-3
            b = _Bucket(buf, 0)
            for _ in range(10):
                global_qsgd_hook(state, b).wait()
            torch.cuda.synchronize()
            # the four library launches of one bucket alone, as graph replays
            dev_us = _hook_device_us(torch, stream, state, buf, steps)
            t0 = time.perf_counter()
            for _ in range(steps):
                fut = global_qsgd_hook(state, b)
            fut.wait()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) / steps * 1e6
            lat = []
            for _ in range(min(steps, 20)):
                t0 = time.perf_counter()
                global_qsgd_hook(state, b).wait()
                torch.cuda.synchronize()
                lat.append(time.perf_counter() - t0)
            out[label] = {"elements": buf.numel(), "us": round(us, 2),
                          "bucket_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "latency_us": round(1e6 * sorted(lat)[len(lat) // 2], 1),
                          "device_us": round(dev_us, 2)}
            del buf
    finally:
        dist.destroy_process_group()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the n workers are "
              "simulated as rows of one device buffer and the library has no collective",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import allreduce_compatible_gradient_amd as gq
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        nbytes = 1 << 30
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}))
        return

    w = wl.WORKLOADS[args.workload]
    xd, gen_s = load_workload(np, torch, wl, w, dev)
    n, d = w.n, w.d
    t = time_workload(gq, np, torch, w, xd, stream, args.steps, args.warmup, full=True)
    mean, norm, ws, ms = t.pop("_mean"), t.pop("_norm"), t.pop("_ws"), t["ms_per_step"]
    in_bytes = n * d * w.elem_bytes
    W = gq.gq_min_code_bits(n, w.s, w.scheme)
    out = {
        "metric": "fused Global-QSGD compress+int-sum+dequant GB/s (fp32 in) and % HBM peak",
        "value": t["input_GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": workload_config(w, W),
        "hbm_frac_fused": t["hbm_frac_fused"],
        "graph_replay": t["graph_replay"],
        "cold_cache": t["cold_cache"],
        "kernels_ms": t["kernels_ms"],
        "compress_step": t["compress_step"],
        "roofline": t["roofline"],
        "bits_per_element": w.code_bits,
        "input_gen_s": round(gen_s, 2),
    }
    # ---- the measured read ceiling: the best plain stream read of this input
    # (probe kernels in several launch shapes, and the library's own norm
    # pass, which reads the same bytes and nothing else)
    from allreduce_compatible_gradient_amd import probe
    if not args.no_extras:
        rc = probe.read_ceiling(xd, reps=5, stream=stream)
        norm_gbs = in_bytes / (t["kernels_ms"]["norm_pass"] * 1e-3) / 1e9
        rc["norm_pass_GBs"] = round(norm_gbs, 1)
        if norm_gbs > rc["GBs"]:
            rc["GBs"], rc["shape"] = round(norm_gbs, 1), "the norm pass (read-only)"
            rc["frac_of_8TBs"] = round(norm_gbs / HBM_PEAK_GBS, 4)
        out["read_ceiling"] = rc
        if out["roofline"]["bound"] == "hbm":
            out["roofline"]["frac_of_read_ceiling"] = round(out["roofline"]["achieved"] / rc["GBs"], 4)
        out["frac_of_read_ceiling_fused"] = round(
            (2 * in_bytes + 4 * d) / (ms * 1e-3) / 1e9 / rc["GBs"], 4)
    if args.unfused:
        def unfused_at(W, reps):
            codes = torch.empty((n, gq.gq_code_row_bytes(d, W)), dtype=torch.uint8, device=dev)
            csum = torch.empty(gq.gq_code_row_bytes(d, W), dtype=torch.uint8, device=dev)

            def ustep():
                gq.gq_global_norm(xd, w.q, w.p, norm=norm, workspace=ws, stream=stream)
                gq.gq_quantize(xd, w.s, w.scheme, norm, w.seed, W, codes=codes, stream=stream)
                gq.gq_reduce_codes(codes, n, d, W, code_sum=csum, stream=stream)
                gq.gq_dequantize(csum, n, d, w.s, w.scheme, W, norm, mean=mean, stream=stream)
            for _ in range(3):
                ustep()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                ustep()
            e1.record(stream)
            torch.cuda.synchronize()
            ums = e0.elapsed_time(e1) / reps
            del codes, csum
            return {"ms_per_step": round(ums, 6), "input_GBs": round(in_bytes / (ums * 1e-3) / 1e9, 3),
                    "code_bits": W}
        out["unfused"] = unfused_at(w.code_bits, args.steps)
        wmin = gq.gq_min_code_bits(n, w.s, w.scheme)
        if wmin != w.code_bits:
            # the same pipeline with codes packed to the minimal width
            out["unfused_min_width"] = unfused_at(wmin, args.steps)
    if args.words:
        gq.gq_global_norm(xd, w.q, w.p, norm=norm, workspace=ws, stream=stream)
        out["words"] = words_report(gq, torch, w, xd, stream, min(args.steps, 50), norm, mean)
    if args.bucket:
        out["bucket"] = bucket_report(gq, torch, w, xd, stream, min(args.steps, 100))
    if args.e8:
        out["e8"] = e8_report(gq, torch, w, xd, stream, min(args.steps, 50), ws)
    if args.ablation or w.key == 5:
        out["ablation"] = ablation(gq, torch, w, xd, stream, args.steps, ms, mean, norm, ws)
    del xd, mean, norm, ws
    torch.cuda.empty_cache()

    # ---- the other large workloads, each whole step and each pass timed the same way
    keys = [int(k) for k in args.configs.split(",") if k.strip() and int(k) != w.key]
    if keys:
        out["configs"] = {}
        for key in keys:
            wk = wl.WORKLOADS[key]
            xk, _ = load_workload(np, torch, wl, wk, dev)
            tk = time_workload(gq, np, torch, wk, xk, stream, max(10, min(args.steps, 50)),
                               min(args.warmup, 5), full=False)
            for k in ("_mean", "_norm", "_ws"):
                del tk[k]
            tk["config"] = workload_config(wk, gq.gq_min_code_bits(wk.n, wk.s, wk.scheme))
            out["configs"][wk.name] = tk
            del xk
            torch.cuda.empty_cache()

    # ---- the pages' 8-bit custom reduction against an fp32 sum (omega), and
    # the measured issue rates behind the VALU-bound kernels' ALU roofline
    if args.valu_probe and args.no_extras:
        out["valu_ceiling"] = probe.valu_rates(stream=stream)
    if not args.no_extras:
        out["e8_omega"] = e8_omega(gq, torch, stream, dev)
        out["valu_ceiling"] = probe.valu_rates(stream=stream)
        try:
            out["ddp_hook"] = ddp_hook_report(torch, w, stream, min(args.steps, 50))
        except Exception as e:  # the record keeps the headline even if RCCL cannot start here
            out["ddp_hook"] = {"error": f"{type(e).__name__}: {e}"}
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
