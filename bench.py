#!/usr/bin/env python3
"""Throughput of one tensor-parallel step on one MI355X.

A step is one pass of the whole hot path over the Llama-3-70B-shaped
workload (T = 16384 tokens, d = 8192, d_ff = 28672, T_p = 8; 64 query / 8 KV
heads of 128): for every rank t of the T_p ranks held on this one GPU,
    column-parallel GEMM  H(t) = silu(X W1(t)) * (X W3(t))   (activation fused)
    row-parallel GEMM     y(t) = H(t) W2(t)                   (partial sum)
then the local partial sum y = sum_t y(t) standing in for the all-reduce; then
the row-sharded attention output projection a(t) = O(t) Wo(t) for every rank
and its partial sum.  Inputs are seeded synthetic tensors resident in HBM
before timing starts.

Prints one JSON line.  value = algorithmic GEMM FLOPs of the step (2MNK per
product) / measured step time.  Per-kernel durations come from HIP events
recorded between the kernels on the stream they run on; the roofline object
describes the dominant kernel (the column-parallel GEMM with the SwiGLU
epilogue).  The CPU baseline is the float64 oracle timed on a bounded sample of
the same workload (a subset of token rows, all ranks), and the sampled rows of
the GPU result are compared with it (max_err).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_SCLK_MHZ = 2400          # the shader clock that peak assumes
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TOL = 2e-2                    # normwise max relative error, bf16 with fp32 accumulation
PSUM_PAD = 2048               # elements between partial slices (4 KiB of bf16)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Sources the column GEMM is built from: the committed HBM traffic describes this kernel
# only while they are unchanged.
GEMM_SOURCES = ("gemm_bf16.hip", "lds_copy.h", "tp_internal.h")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "megatron_tensor_transformer_gemm_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, path: str | None = None):
    """HBM traffic of the dominant kernel from the committed PMC summary, if it still
    describes the current kernel sources (else None)."""
    path = path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("kernels", {}).get(f"{kernel}@{workload}")
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("bytes_per_launch")


def column_gemm_traffic_bounds(T: int, d: int, n: int) -> tuple:
    """Bytes per launch of the gated column GEMM (bf16 X [T, d] times the W1 and W3 column
    blocks [d, n], H [T, n] written): the compulsory bytes, and the bytes the persistent
    256 x 256 tiling implies.  Each XCD's 32 concurrent tiles form a 4 x 8 block whose
    k-sweep streams 4 A and 8 B panels (256 x d each) through the XCD's L2, once per sweep
    of 256 tiles; H is written once.  (The model is for products of whole sweeps, such as
    the 70B shard's 1,792 tiles.)"""
    compulsory = 2 * (T * d + 2 * d * n + T * n)
    tiles = -(-T // 256) * -(-(2 * n) // 256)
    sweeps = -(-tiles // 256)
    model = sweeps * 8 * (4 + 8) * (256 * d * 2) + 2 * T * n
    return compulsory, model


def host_cpu_info() -> dict:
    """The host's CPU model, its physical cores and the logical CPUs this process may use
    (from /proc/cpuinfo and the affinity mask)."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "physical_cores": len(cores) or None, "usable_logical_cpus": usable}


def percentiles(vals) -> dict:
    """Median, p10 and p90 of a list of durations (nearest-rank)."""
    v = sorted(vals)

    def at(q):
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"median": at(0.5), "p10": at(0.1), "p90": at(0.9), "calls": len(v)}


class SclkSampler:
    """Samples the shader clock from a host thread while the GPU works: the current DPM
    level (the line marked '*') of the card's pp_dpm_sclk, every `period_s` seconds.
    Reports nothing when there is not exactly one card or the file cannot be read."""

    def __init__(self, period_s: float = 0.01):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if len(paths) == 1 else None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        import re
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1],
                "samples": len(v),
                "source": "current DPM level in pp_dpm_sclk, sampled every "
                          f"{int(self.period * 1e3)} ms over the timed steps"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="token rows of the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the extra GPT-style block measurement (attention core)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the extra measurement of the FFN shard backward")
    ap.add_argument("--no-ring", action="store_true",
                    help="skip the extra measurement of ring attention (context parallelism)")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the vendor-library reference (torch.matmul) on the same products")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the extra measurement of the smaller FFN workloads (configs 1-3)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="read the rocprofv3 counter_collection.csv files of two --pmc-pass "
                         "runs (FETCH_SIZE, WRITE_SIZE), write profiles/hbm_traffic.json, exit")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run each kernel of one step once, then a plain 1 GiB device copy "
                         "(the calibration for the HBM byte counters), and exit")
    args = ap.parse_args()

    if args.ingest_pmc:
        return ingest_pmc(*args.ingest_pmc)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU: every tensor-parallel "
                                   "rank's shard runs on that GPU and a local partial sum stands "
                                   "in for the all-reduce; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import numpy as np
    import torch

    from megatron_tensor_transformer_gemm_amd import inputs as I
    from megatron_tensor_transformer_gemm_amd import tpshard as S

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    torch.cuda.set_device(0)
    S.lib()  # fail now if the HIP library is not built

    w = I.WORKLOADS[4]
    T, d, d_ff, T_p = w.T, w.d, w.d_ff, w.T_p
    n = d_ff // T_p
    h_t = w.n_heads // T_p
    kdim = h_t * w.head_dim
    log(f"[bench] workload {w.name}: T={T} d={d} d_ff={d_ff} T_p={T_p}; generating inputs")
    t0 = time.perf_counter()
    host = {k: I.make_tensor(w, k) for k in ("x", "w1", "w3", "w2", "wo", "o")}

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    X, W1, W3, W2, WO = (dev(host[k]) for k in ("x", "w1", "w3", "w2", "wo"))
    O_t = [dev(host["o"][:, t * kdim:(t + 1) * kdim]) for t in range(T_p)]
    H = torch.empty((T, n), dtype=torch.bfloat16, device="cuda")
    # Partial buffer: slice t holds y(t) [T, d]; the slices are padded by 4 KiB so that the
    # same element of every slice does not fall on the same DRAM banks (the slice size,
    # 2^28 bytes here, is a power of two).
    stride = T * d + PSUM_PAD
    P_flat = torch.empty(T_p * stride, dtype=torch.bfloat16, device="cuda")
    P = [P_flat[t * stride: t * stride + T * d].view(T, d) for t in range(T_p)]
    Y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    A = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")

    BF = S.TP_BF16
    n_kernels = 2 * T_p + 1 + T_p + 1
    names = []
    for _ in range(T_p):
        names += ["col", "row"]
    names += ["psum"] + ["outproj"] * T_p + ["psum"]
    assert len(names) == n_kernels

    def step(evs=None):
        k = 0
        if evs:
            evs[0].record()
        for t in range(T_p):
            S.tp_ffn_column_fwd(X, W1, W3, H, T, d, d_ff, T_p, t, S.TP_ACT_SWIGLU, BF)
            if evs:
                k += 1
                evs[k].record()
            S.tp_ffn_row_fwd(H, W2, P[t], T, d, d_ff, T_p, t, BF, BF)
            if evs:
                k += 1
                evs[k].record()
        S.tp_partial_sum(P_flat, stride, T_p, None, Y, T * d, BF, BF)
        if evs:
            k += 1
            evs[k].record()
        for t in range(T_p):
            S.tp_attn_outproj_shard_fwd(O_t[t], WO, P[t], T, d, w.n_heads, w.n_kv_heads,
                                        w.head_dim, T_p, t, BF, BF)
            if evs:
                k += 1
                evs[k].record()
        S.tp_partial_sum(P_flat, stride, T_p, None, A, T * d, BF, BF)
        if evs:
            k += 1
            evs[k].record()

    if args.pmc_pass:
        # one launch of each kernel class, then a copy of known size
        S.tp_ffn_column_fwd(X, W1, W3, H, T, d, d_ff, T_p, 0, S.TP_ACT_SWIGLU, BF)
        S.tp_ffn_row_fwd(H, W2, P[0], T, d, d_ff, T_p, 0, BF, BF)
        S.tp_partial_sum(P_flat, stride, T_p, None, Y, T * d, BF, BF)
        S.tp_attn_outproj_shard_fwd(O_t[0], WO, P[0], T, d, w.n_heads, w.n_kv_heads, w.head_dim,
                                    T_p, 0, BF, BF)
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")  # 1 GiB
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] pmc pass done: column GEMM, row GEMM, partial sum, out-projection, "
            "1 GiB copy")
        return 0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_kernels + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    with SclkSampler() as sclk_sampler:
        t_start = time.perf_counter()
        for s in range(args.steps):
            step(ev[s])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    sclk = sclk_sampler.summary()
    ms_per_step = elapsed * 1e3 / args.steps

    dur = {}  # kernel name -> list of ms
    for s in range(args.steps):
        for i, nm in enumerate(names):
            dur.setdefault(nm, []).append(ev[s][i].elapsed_time(ev[s][i + 1]))
    avg_us = {k: 1e3 * sum(v) / len(v) for k, v in dur.items()}
    step_ms_each = [round(ev[s][0].elapsed_time(ev[s][n_kernels]), 3) for s in range(args.steps)]

    fl_col = 2.0 * T * d * n * 2
    fl_row = 2.0 * T * n * d
    fl_out = 2.0 * T * kdim * d
    step_flops = T_p * (fl_col + fl_row + fl_out)
    psum_bytes = (T_p + 1) * T * d * 2
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s")

    def tfl(fl, us):
        return fl / (us * 1e-6) / 1e12

    kernels = {
        "column_gemm_swiglu": {"avg_us": round(avg_us["col"], 2),
                               "tflops": round(tfl(fl_col, avg_us["col"]), 1),
                               "frac_peak": round(tfl(fl_col, avg_us["col"]) / PEAK_BF16_TFLOPS, 4),
                               "launches_per_step": T_p},
        "row_gemm": {"avg_us": round(avg_us["row"], 2),
                     "tflops": round(tfl(fl_row, avg_us["row"]), 1),
                     "frac_peak": round(tfl(fl_row, avg_us["row"]) / PEAK_BF16_TFLOPS, 4),
                     "launches_per_step": T_p},
        "attn_outproj_gemm": {"avg_us": round(avg_us["outproj"], 2),
                              "tflops": round(tfl(fl_out, avg_us["outproj"]), 1),
                              "frac_peak": round(tfl(fl_out, avg_us["outproj"]) / PEAK_BF16_TFLOPS, 4),
                              "launches_per_step": T_p},
        "partial_sum": {"avg_us": round(avg_us["psum"], 2),
                        "gbs": round(psum_bytes / (avg_us["psum"] * 1e-6) / 1e9, 1),
                        "frac_peak": round(psum_bytes / (avg_us["psum"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "launches_per_step": 2},
    }
    col_tf = tfl(fl_col, avg_us["col"])
    roofline = {"bound": "mfma", "achieved": round(col_tf, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(col_tf / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic("column_gemm_swiglu", w.name),
                "kernel": "column-parallel GEMM + SwiGLU epilogue (per rank)",
                "flops_per_launch": fl_col}
    # what `traffic` compares with: the bytes the kernel must move, and what its tiling
    # streams from beyond L2 at best (the rest is workgroups drifting apart)
    roofline["traffic_compulsory"], roofline["traffic_tiling_model"] = column_gemm_traffic_bounds(T, d, n)
    if sclk:
        # the same kernel against the MFMA rate at the clock the power manager set
        roofline["frac_at_measured_sclk"] = round(
            col_tf / (PEAK_BF16_TFLOPS * sclk["median_mhz"] / PEAK_SCLK_MHZ), 4)
        log(f"[bench] shader clock over the timed steps: median {sclk['median_mhz']} MHz "
            f"({sclk['min_mhz']}-{sclk['max_mhz']}, {sclk['samples']} samples)")

    out = {
        "metric": "TP-shard FFN fwd TFLOP/s (bf16, 1 GPU) + % of MFMA peak; oracle-match max err",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "T": T, "d": d, "d_ff": d_ff, "T_p": T_p,
                   "ranks_per_step": T_p, "act": "swiglu", "n_heads": w.n_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "parallelism": f"tp{T_p} ranks emulated on 1 GPU"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "step_gemm_flops": step_flops,
        "kernels": kernels,
        "step_ms_each": step_ms_each,
        "roofline": roofline,
        "sclk": sclk,
    }

    # sequence-parallel form of the same reduce: 8 ranks' row slices (reduce-scatter), into
    # a buffer of its own (Y and A keep the step's results for the CPU comparison)
    Yrs = torch.empty_like(Y)
    rs_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rs_reps = 5
    for _ in range(2):
        for t in range(T_p):
            S.tp_reduce_scatter_rows(P_flat, stride, T_p, t, None, Yrs[t * (T // T_p):], T, d, BF, BF)
    rs_ev[0].record()
    for _ in range(rs_reps):
        for t in range(T_p):
            S.tp_reduce_scatter_rows(P_flat, stride, T_p, t, None, Yrs[t * (T // T_p):], T, d, BF, BF)
    rs_ev[1].record()
    torch.cuda.synchronize()
    # the gathered rows are the full sum of the same partials (the out-projection's, A)
    out_rs_equal = bool(torch.equal(Yrs, A))
    del Yrs
    rs_us = 1e3 * rs_ev[0].elapsed_time(rs_ev[1]) / rs_reps
    out["sequence_parallel"] = {
        "what": "reduce-scatter of the 70B y(t) partials: each of 8 ranks sums its 2048 token rows",
        "all_ranks_us": round(rs_us, 1), "per_rank_us": round(rs_us / T_p, 1),
        "gbs": round(psum_bytes / (rs_us * 1e-6) / 1e9, 1),
        "full_partial_sum_us": round(avg_us["psum"], 1),
        "rows_equal_full_sum": out_rs_equal}
    log(f"[bench] reduce-scatter: 8 ranks {rs_us:.1f} us (full sum {avg_us['psum']:.1f} us)")

    out["shard_fwd_calls"] = measure_shard_calls(S, w, X, W1, W3, W2, H, P, 50)
    if not args.no_vendor:
        out["vendor_reference"] = measure_vendor(S, w, X, W1, W3, W2, H, O_t[0], WO, P[0],
                                                 max(4, args.steps // 2))
    if not args.no_backward:
        out["backward"] = measure_backward(w, X, W1, W3, W2, max(2, args.steps // 4), 1)
    if not args.no_block:
        out["block_workload"] = measure_block(max(2, args.steps // 4), 1)
    if not args.no_ring:
        out["context_parallel_ring"] = measure_ring(max(2, args.steps // 4), 1)
    cfg_outputs = None
    if not args.no_configs:
        out["configs"], cfg_outputs = measure_configs(max(8, args.steps), 2)
    if not args.no_cpu_baseline:
        out.update(cpu_baseline(host, w, Y, A, args.cpu_rows))
        if cfg_outputs:
            cpu_check_configs(out["configs"], cfg_outputs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    failures = parity_failures(out)
    if failures:
        log("[bench] PARITY FAILURE in: " + ", ".join(failures))
        return 3
    return 0


def parity_failures(out: dict) -> list:
    """Names of the checks in the result that did not meet their tolerance."""
    bad = []
    if out.get("max_err") and not out["max_err"].get("pass", False):
        bad.append("max_err")
    for name, r in (out.get("configs") or {}).items():
        if "pass" in r and not r["pass"]:
            bad.append(f"configs.{name}")
    ring = out.get("context_parallel_ring")
    if ring and not ring["max_err_vs_whole"] <= TOL:
        bad.append("context_parallel_ring")
    sp = out.get("sequence_parallel")
    if sp and not sp["rows_equal_full_sum"]:
        bad.append("sequence_parallel")
    return bad


def measure_shard_calls(S, w, X, W1, W3, W2, H, P, calls: int) -> dict:
    """Per-call duration of tp_ffn_shard_fwd (column GEMM + SwiGLU, row GEMM) at the
    headline shape: `calls` calls cycling over the ranks, each between its own pair of HIP
    events on the launch stream; median and p10/p90."""
    import torch

    T, d, d_ff, T_p = w.T, w.d, w.d_ff, w.T_p
    n = d_ff // T_p
    BF = S.TP_BF16
    nb = S.tp_ffn_workspace_bytes(T, d_ff, T_p, BF)
    ws = H.view(torch.uint8).view(-1)
    assert ws.numel() >= nb
    for t in range(2):
        S.tp_ffn_shard_fwd(X, W1, W3, W2, P[t], ws, nb, T, d, d_ff, T_p, t, "swiglu", BF, BF)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    torch.cuda.synchronize()
    for i in range(calls):
        t = i % T_p
        ev[i][0].record()
        S.tp_ffn_shard_fwd(X, W1, W3, W2, P[t], ws, nb, T, d, d_ff, T_p, t, "swiglu", BF, BF)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = [1e3 * a.elapsed_time(b) for a, b in ev]
    st = percentiles(us)
    fl = 2.0 * T * d * n * 2 + 2.0 * T * n * d
    res = {"what": f"{w.name}: tp_ffn_shard_fwd, one rank's whole FFN shard per call",
           "median_us": round(st["median"], 1), "p10_us": round(st["p10"], 1),
           "p90_us": round(st["p90"], 1), "calls": st["calls"],
           "median_tflops": round(fl / (st["median"] * 1e-6) / 1e12, 1),
           "median_frac_peak": round(fl / (st["median"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "flops_per_call": fl}
    log(f"[bench] shard fwd calls: median {st['median']:.1f} us (p10 {st['p10']:.1f}, "
        f"p90 {st['p90']:.1f}), {res['median_tflops']} TFLOP/s")
    return res


PMC_PASS_KERNELS = ["column_gemm_swiglu", "row_gemm", "partial_sum", "attn_outproj_gemm"]


def ingest_pmc(fetch_csv: str, write_csv: str, out_path: str | None = None) -> int:
    """Per-launch HBM bytes of each kernel of the --pmc-pass run.

    FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  Each is scaled by
    (bytes a plain 1 GiB copy really moves) / (what the same counter reads for that copy).
    Dispatch order of --pmc-pass: column GEMM, row GEMM, partial sum, out-projection,
    fill, copy."""
    import csv

    def per_dispatch(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]

    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    f_copy = [v for n, v in fetch if "copy" in n.lower()][-1] * 1024.0
    w_copy = [v for n, v in write if "copy" in n.lower()][-1] * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    out = {"workload": "llama3_70b_swiglu_bf16", "source_digest": kernel_source_digest(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_counted": f_copy,
                           "write_counted": w_copy, "fetch_scale": f_scale,
                           "write_scale": w_scale},
           "kernels": {}}
    for i, name in enumerate(PMC_PASS_KERNELS):
        fb = fetch[i][1] * 1024.0 * f_scale
        wb = write[i][1] * 1024.0 * w_scale
        out["kernels"][f"{name}@llama3_70b_swiglu_bf16"] = {
            "kernel_symbol": fetch[i][0], "fetch_bytes": fb, "write_bytes": wb,
            "bytes_per_launch": fb + wb, "source_digest": out["source_digest"]}
    path = out_path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out["kernels"], indent=1))
    return 0


def measure_vendor(S, w, X, W1, W3, W2, H, O0, WO, Y0, steps) -> dict:
    """The vendor library beside this library on rank 0's products of the 70B step, both
    timed the same way: one product repeated on the same operands, events on the current
    stream, after the step's timed region.  The library is torch.matmul (hipBLASLt on
    ROCm) on the same bf16 operands and layouts (weight blocks as strided slices of the
    full matrices); it runs the column product as two plain products X W1(0), X W3(0)
    without the activation.  Repeating one product keeps its operands in the 256 MB MALL,
    so these times are shorter than inside the step, where every rank reads its own
    blocks."""
    import torch

    T, d, d_ff, T_p = w.T, w.d, w.d_ff, w.T_p
    n, kdim = d_ff // T_p, (w.n_heads // T_p) * w.head_dim
    BF = S.TP_BF16
    U = torch.empty((T, n), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(U)
    W1b, W3b, W2b, WOb = W1[:, :n], W3[:, :n], W2[:n, :], WO[:kdim, :]
    prods = {
        "column_gemm_swiglu": (
            lambda: S.tp_ffn_column_fwd(X, W1, W3, H, T, d, d_ff, T_p, 0, S.TP_ACT_SWIGLU, BF),
            lambda: (torch.matmul(X, W1b, out=U), torch.matmul(X, W3b, out=V)),
            2 * 2.0 * T * d * n),
        "row_gemm": (
            lambda: S.tp_ffn_row_fwd(H, W2, Y0, T, d, d_ff, T_p, 0, BF, BF),
            lambda: torch.matmul(H, W2b, out=Y0), 2.0 * T * n * d),
        "attn_outproj_gemm": (
            lambda: S.tp_attn_outproj_shard_fwd(O0, WO, Y0, T, d, w.n_heads, w.n_kv_heads,
                                                w.head_dim, T_p, 0, BF, BF),
            lambda: torch.matmul(O0, WOb, out=Y0), 2.0 * T * kdim * d),
    }

    def timed(fn):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    res = {"library": "torch.matmul (hipBLASLt), same operands; its column product is two "
                      "plain products without the activation",
           "timing": "one product repeated on the same operands (MALL-resident), both sides"}
    for name, (ours, vendor, fl) in prods.items():
        t_o, t_v = timed(ours), timed(vendor)
        t_o2 = timed(ours)   # again, so that neither side always runs on the colder chip
        t_o = min(t_o, t_o2)
        res[name] = {"ours_us": round(t_o, 1), "ours_tflops": round(fl / t_o / 1e6, 1),
                     "vendor_us": round(t_v, 1), "vendor_tflops": round(fl / t_v / 1e6, 1),
                     "ours_over_vendor_time": round(t_o / t_v, 3)}
        log(f"[bench] {name}, repeated: ours {t_o:.1f} us, vendor {t_v:.1f} us")
    return res


def measure_backward(w, X, W1, W3, W2, steps: int, warmup: int) -> dict:
    """Backward of the FFN sublayer's TP shards at the headline shape, all ranks: per rank
    tp_ffn_shard_bwd (dU/dV with the SwiGLU derivative, dW2, dX(t), dW1|dW3), then the
    partial sum of the ranks' dX(t) (the f all-reduce).  The ranks' saved activations (H, U,
    V from the training forward) are made before the timed region.  Algorithmic FLOPs per
    rank: 2*T*d*n for dH, dW2 each, 4*T*d*n for dX and for dW1|dW3 (gated)."""
    import numpy as np
    import torch

    from megatron_tensor_transformer_gemm_amd import inputs as I
    from megatron_tensor_transformer_gemm_amd import tpshard as S

    torch.cuda.empty_cache()
    T, d, d_ff, T_p = w.T, w.d, w.d_ff, w.T_p
    n = d_ff // T_p
    BF, F32 = S.TP_BF16, S.TP_F32
    log(f"[bench] backward {w.name}: saved activations of {T_p} ranks")
    dy = torch.from_numpy(np.ascontiguousarray(I.make_tensor(w, "dy")).view(np.int16)).view(
        torch.bfloat16).cuda()
    saved = []
    yt = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    for t in range(T_p):
        h, u, v = (torch.empty((T, n), dtype=torch.bfloat16, device="cuda") for _ in range(3))
        S.tp_ffn_shard_fwd_train(X, W1, W3, W2, yt, h, u, v, T, d, d_ff, T_p, t, S.TP_ACT_SWIGLU, BF)
        saved.append((h, u, v))
    # the training forward itself (it keeps H, U, V): every rank's call between events,
    # after one untimed pass
    fwd_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(2 * T_p)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(fwd_ev):
        t = i % T_p
        h, u, v = saved[t]
        e0.record()
        S.tp_ffn_shard_fwd_train(X, W1, W3, W2, yt, h, u, v, T, d, d_ff, T_p, t, S.TP_ACT_SWIGLU, BF)
        e1.record()
    torch.cuda.synchronize()
    fwd_us = 1e3 * sum(a.elapsed_time(b) for a, b in fwd_ev) / len(fwd_ev)
    del yt
    dW1 = torch.empty((d, d_ff), dtype=torch.float32, device="cuda")
    dW3 = torch.empty((d, d_ff), dtype=torch.float32, device="cuda")
    dW2 = torch.empty((d_ff, d), dtype=torch.float32, device="cuda")
    stride = T * d + PSUM_PAD
    Pf = torch.empty(T_p * stride, dtype=torch.bfloat16, device="cuda")
    P = [Pf[t * stride: t * stride + T * d].view(T, d) for t in range(T_p)]
    dX = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    nb = S.tp_ffn_bwd_workspace_bytes(T, d_ff, T_p, S.TP_ACT_SWIGLU)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step(evs=None):
        if evs:
            evs[0].record()
        for t in range(T_p):
            h, u, v = saved[t]
            S.tp_ffn_shard_bwd(X, W1, W3, W2, dy, h, u, v, P[t], dW1, dW3, dW2, ws, nb, T, d, d_ff,
                               T_p, t, S.TP_ACT_SWIGLU, BF, F32)
            if evs:
                evs[t + 1].record()
        S.tp_partial_sum(Pf, stride, T_p, None, dX, T * d, BF, BF)
        if evs:
            evs[T_p + 1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(T_p + 2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(ev[s_])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    rank_us = 1e3 * sum(e[t].elapsed_time(e[t + 1]) for e in ev for t in range(T_p)) / (steps * T_p)
    psum_us = 1e3 * sum(e[T_p].elapsed_time(e[T_p + 1]) for e in ev) / steps
    fl_rank = 12.0 * T * d * n
    res = {"workload": f"{w.name} backward: {T_p} ranks' tp_ffn_shard_bwd + partial sum of dX",
           "ms_per_step": round(ms, 3),
           "tflops": round(T_p * fl_rank / (ms * 1e-3) / 1e12, 1),
           "frac_of_peak": round(T_p * fl_rank / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "per_rank_us": round(rank_us, 1),
           "per_rank_tflops": round(fl_rank / (rank_us * 1e-6) / 1e12, 1),
           "flops_per_rank": fl_rank,
           "dx_partial_sum_us": round(psum_us, 1),
           "dtypes": {"inputs": "bf16", "dx": "bf16", "weight_grads": "f32"},
           "steps": steps,
           "train_forward": {"what": "tp_ffn_shard_fwd_train of one rank: the forward shard that "
                                     "also keeps H, U, V for the backward",
                             "per_rank_us": round(fwd_us, 1),
                             "tflops": round(6.0 * T * d * n / (fwd_us * 1e-6) / 1e12, 1),
                             "calls": len(fwd_ev)}}
    log(f"[bench] backward: {ms:.3f} ms/step, {res['tflops']} TFLOP/s; per rank {rank_us:.1f} us; "
        f"training forward per rank {fwd_us:.1f} us")
    return res


def measure_block(steps: int, warmup: int) -> dict:
    """GPT-style TP8 block (d=6144, 48 heads of 128, d_ff=24576, GELU), 4 micro-batches of one
    2048-token sequence, all ranks: per rank QKV projections + causal attention core +
    out-projection, reduce with residual, per rank column + row GEMM, reduce with residual.
    Reports the block's GEMM+attention FLOP rate and per-kernel times, including the
    attention core alone (causal FLOPs 2*h_t*d_h*L*(L+1) per rank and sequence)."""
    import numpy as np
    import torch

    from megatron_tensor_transformer_gemm_amd import inputs as I
    from megatron_tensor_transformer_gemm_amd import tpshard as S

    torch.cuda.empty_cache()
    w = I.WORKLOADS[5]
    T_p, d, L, H, dh = w.T_p, w.d, w.seq_len, w.n_heads, w.head_dim
    h_t = H // T_p
    n = w.d_ff // T_p
    kdim = h_t * dh
    BF = S.TP_BF16
    log(f"[bench] block workload {w.name}: generating inputs")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    Wd = {k: dev(I.make_tensor(w, k)) for k in ("wq", "wk", "wv", "wo", "w1", "w2")}
    X = dev(I.make_tensor(w, "x"))
    stride = L * d + PSUM_PAD
    Pf = torch.empty(T_p * stride, dtype=torch.bfloat16, device="cuda")
    P = [Pf[t * stride: t * stride + L * d].view(L, d) for t in range(T_p)]
    o_t = torch.empty((L, kdim), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(S.tp_attn_heads_workspace_bytes(1, L, H, H, dh, T_p), dtype=torch.uint8,
                     device="cuda")
    nbf = S.tp_ffn_workspace_bytes(L, w.d_ff, T_p, BF)   # H(t) and the split-K scratch
    wsf = torch.empty(nbf, dtype=torch.uint8, device="cuda")
    x1 = torch.empty((L, d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((w.T, d), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    names = []
    for _ in range(w.n_seq):
        names += ["attn_heads", "outproj"] * T_p + ["psum"] + ["ffn"] * T_p + ["psum"]

    def step(evs=None):
        k = [0]

        def mark():
            if evs:
                k[0] += 1
                evs[k[0]].record()
        if evs:
            evs[0].record()
        for s_ in range(w.n_seq):
            xs = X[s_ * L:(s_ + 1) * L]
            for t in range(T_p):
                S.tp_attn_heads_shard_fwd(xs, Wd["wq"], Wd["wk"], Wd["wv"], o_t, ws, ws.numel(), 1, L,
                                          d, H, H, dh, T_p, t, True)
                mark()
                S.tp_attn_outproj_shard_fwd(o_t, Wd["wo"], P[t], L, d, H, H, dh, T_p, t, BF, BF)
                mark()
            S.tp_partial_sum(Pf, stride, T_p, xs, x1, L * d, BF, BF)
            mark()
            for t in range(T_p):
                S.tp_ffn_shard_fwd(x1, Wd["w1"], None, Wd["w2"], P[t], wsf, nbf, L, d, w.d_ff, T_p, t,
                                   S.TP_ACT_GELU, BF, BF)
                mark()
            S.tp_partial_sum(Pf, stride, T_p, x1, y[s_ * L:(s_ + 1) * L], L * d, BF, BF)
            mark()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(ev[s_])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    dur = {}
    for s_ in range(steps):
        for i, nm in enumerate(names):
            dur.setdefault(nm, []).append(ev[s_][i].elapsed_time(ev[s_][i + 1]))
    avg = {k: 1e3 * sum(v) / len(v) for k, v in dur.items()}

    ms_graph = graph_replay_ms(step, steps)
    # the attention core alone, on the last rank's projected heads: 20 calls in one graph
    q = ws.view(torch.bfloat16)
    qv = q[: L * kdim]
    kv = q[L * kdim: 2 * L * kdim]
    vv = q[2 * L * kdim: 3 * L * kdim]

    def cores():
        for _ in range(20):
            S.tp_attn_core_fwd(qv, kv, vv, o_t, 1, L, h_t, h_t, dh, kdim, kdim, kdim, True)
    core_us = graph_replay_ms(cores, 5) * 1e3 / 20
    fl_qkv = 2.0 * L * d * 3 * kdim
    fl_core = 2.0 * h_t * dh * L * (L + 1)
    fl_out = 2.0 * L * kdim * d
    fl_ffn1 = 2.0 * L * d * n
    fl_ffn2 = 2.0 * L * n * d
    fl_step = w.n_seq * T_p * (fl_qkv + fl_core + fl_out + fl_ffn1 + fl_ffn2)

    def tf(fl, us):
        return round(fl / (us * 1e-6) / 1e12, 1)
    res = {
        "workload": w.name, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_graph, 4),
        "timing": "graph replay of the whole step (per-kernel times below: eager, HIP events)",
        "tflops": round(fl_step / (ms_graph * 1e-3) / 1e12, 2), "step_flops": fl_step,
        "eager_ms_per_step": round(ms, 4), "eager_tflops": round(fl_step / (ms * 1e-3) / 1e12, 2),
        "kernels": {
            "qkv_projection_plus_attention_core": {"avg_us": round(avg["attn_heads"], 2),
                                                   "tflops": tf(fl_qkv + fl_core, avg["attn_heads"])},
            "attention_core_causal": {"avg_us": round(core_us, 2), "tflops": tf(fl_core, core_us),
                                      "timing": "20 calls replayed as one graph",
                                      "frac_peak": round(fl_core / (core_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "attn_outproj_gemm": {"avg_us": round(avg["outproj"], 2), "tflops": tf(fl_out, avg["outproj"])},
            "ffn_shard_gelu": {"avg_us": round(avg["ffn"], 2), "tflops": tf(fl_ffn1 + fl_ffn2, avg["ffn"]),
                               "what": "tp_ffn_shard_fwd: column GEMM + GELU (split-K when it "
                                       "cannot fill the GPU) and row GEMM"},
            "partial_sum_residual": {"avg_us": round(avg["psum"], 2)},
        },
    }
    log(f"[bench] block: {ms_graph:.3f} ms/step as a graph, {res['tflops']} TFLOP/s (eager {ms:.3f} ms); "
        f"attention core {core_us:.1f} us")
    return res


def graph_replay_ms(fn, reps: int, warmup: int = 2) -> float:
    """fn (launches only: no allocation, memset or synchronisation) captured once as a
    graph and replayed `reps` times: GPU time per replay in ms, free of the host's
    per-call overhead, which exceeds some of these kernels."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    for _ in range(warmup):
        graph.replay()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a0.record()
    for _ in range(reps):
        graph.replay()
    a1.record()
    torch.cuda.synchronize()
    return a0.elapsed_time(a1) / reps


def measure_ring(steps: int, warmup: int) -> dict:
    """Context parallelism on one GPU: a rank's 6 heads of 128 (the GPT block's TP8 share)
    over one causal 8192-token sequence split into 4 chunks of 2048.  Every CP rank r sets
    up its running state, folds in K/V chunks r, r-1, ..., 0 (the later ones lie after its
    queries and are skipped), and writes O.  Reported: the four ranks' ring work against
    one attention-core call on the whole sequence (same causal FLOPs), the most loaded
    rank alone (its time is the group's critical path when each rank has a GPU), and the
    normwise difference of the two outputs."""
    import torch

    from megatron_tensor_transformer_gemm_amd import tpshard as S

    L, C, h_t, dh = 8192, 4, 6, 128
    c, kd = L // C, h_t * dh
    g = torch.Generator(device="cuda").manual_seed(11)
    q, k, v = (torch.randn(L, kd, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    o_full = torch.empty(L, kd, dtype=torch.bfloat16, device="cuda")
    o_ring = torch.empty(L, kd, dtype=torch.bfloat16, device="cuda")
    st = [torch.empty(c, kd, dtype=torch.float32, device="cuda") for _ in range(C)]
    lse = [torch.empty(c, h_t + 2, dtype=torch.float32, device="cuda") for _ in range(C)]

    def full():
        S.tp_attn_core_fwd(q, k, v, o_full, 1, L, h_t, h_t, dh, kd, kd, kd, True)

    def ring(ranks=range(C)):
        for r in ranks:
            S.tp_attn_ring_init(st[r], lse[r], c, h_t, dh, kd, h_t + 2)
            for s_ in range(C):
                src = (r - s_) % C
                S.tp_attn_ring_step(q[r * c:], k[src * c:], v[src * c:], st[r], lse[r], 1, c, h_t, h_t,
                                    dh, kd, kd, kd, h_t + 2, r * c, src * c, True)
            S.tp_attn_ring_finish(st[r], o_ring[r * c:], c, h_t, dh, kd, kd)

    def timed(fn):
        for _ in range(warmup + 1):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / steps

    # graph replays (several of these kernels are shorter than a host call), eager beside them
    eager_ring_us = timed(ring)
    full_us = 1e3 * graph_replay_ms(full, steps, warmup)
    last_us = 1e3 * graph_replay_ms(lambda: ring([C - 1]), steps, warmup)   # every chunk visible
    ring_us = 1e3 * graph_replay_ms(ring, steps, warmup)
    ring()
    torch.cuda.synchronize()
    diff = float((o_ring.float() - o_full.float()).abs().max() / o_full.float().abs().max())
    fl = 2.0 * h_t * dh * L * (L + 1)
    log(f"[bench] ring attention: 4 CP ranks {ring_us:.1f} us as a graph (last rank {last_us:.1f} us; "
        f"eager {eager_ring_us:.1f} us) vs whole sequence {full_us:.1f} us, max_err {diff:.2e}")
    if diff > 2e-2:
        log(f"[bench] PARITY FAILURE: ring attention differs from the whole-sequence core by {diff:.3e}")
    return {"what": "causal 8192-token sequence, 6 heads of 128, 4 context-parallel chunks of 2048: "
                    "all ranks' ring steps (init, 10 chunk folds, finish) vs one whole-sequence core call",
            "timing": "graph replays; eager_ring_all_ranks_us: the same calls from the host",
            "ring_all_ranks_us": round(ring_us, 1), "whole_sequence_us": round(full_us, 1),
            "last_rank_us": round(last_us, 1), "eager_ring_all_ranks_us": round(eager_ring_us, 1),
            "ring_tflops": round(fl / (ring_us * 1e-6) / 1e12, 1),
            "whole_tflops": round(fl / (full_us * 1e-6) / 1e12, 1),
            "max_err_vs_whole": diff}


def measure_configs(steps: int, warmup: int):
    """The smaller FFN workloads (tiny fp32 GELU, GPT-2-medium GELU, Llama-3-8B SwiGLU): all
    ranks' tp_ffn_shard_fwd and the partial sum, per step, timed as a replayed graph (and
    eagerly, with per-shard event times, for comparison).  Returns the results and, for the oracle check of the CPU-baseline
    leg, the host inputs and the reduced outputs."""
    import numpy as np
    import torch

    from megatron_tensor_transformer_gemm_amd import inputs as I
    from megatron_tensor_transformer_gemm_amd import tpshard as S

    res, keep = {}, {}
    for cid in (1, 2, 3):
        w = I.WORKLOADS[cid]
        f32 = w.dtype == I.F32
        code = S.TP_F32 if f32 else S.TP_BF16
        tdt = torch.float32 if f32 else torch.bfloat16
        gated = w.act == "swiglu"
        names = ("x", "w1", "w3", "w2") if gated else ("x", "w1", "w2")
        host = {k: I.make_tensor(w, k) for k in names}

        def dev(a):
            if f32:
                return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        X, W1, W2 = dev(host["x"]), dev(host["w1"]), dev(host["w2"])
        W3 = dev(host["w3"]) if gated else None
        T, d, d_ff, T_p = w.T, w.d, w.d_ff, w.T_p
        n = d_ff // T_p
        parts = torch.empty((T_p, T, d), dtype=tdt, device="cuda")
        nb = S.tp_ffn_workspace_bytes(T, d_ff, T_p, code)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
        y = torch.empty((T, d), dtype=tdt, device="cuda")

        def step(evs=None):
            for t in range(T_p):
                if evs:
                    evs[t][0].record()
                S.tp_ffn_shard_fwd(X, W1, W3, W2, parts[t], ws, nb, T, d, d_ff, T_p, t, w.act, code, code)
                if evs:
                    evs[t][1].record()
            S.tp_partial_sum(parts, T * d, T_p, None, y, T * d, code, code)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(T_p)]
              for _ in range(steps)]
        t0 = time.perf_counter()
        for s_ in range(steps):
            step(ev[s_])
        torch.cuda.synchronize()
        ms_eager = (time.perf_counter() - t0) * 1e3 / steps
        shard_calls = [1e3 * e[0].elapsed_time(e[1]) for es in ev for e in es]
        shard_us = sum(shard_calls) / len(shard_calls)
        shard_st = percentiles(shard_calls)
        # Small problems finish before the host submits the next launch: replaying the step
        # as one captured graph times the GPU's work alone.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(warmup):
            graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        fl_shard = 2.0 * T * d * n * (2 if gated else 1) + 2.0 * T * n * d
        peak = PEAK_F32_TFLOPS if f32 else PEAK_BF16_TFLOPS
        tf = T_p * fl_shard / (ms * 1e-3) / 1e12
        res[w.name] = {"act": w.act, "dtype": "f32" if f32 else "bf16", "T": T, "d": d, "d_ff": d_ff,
                       "T_p": T_p, "ms_per_step": round(ms, 4), "timing": "graph replay",
                       "step_tflops": round(tf, 2), "step_frac_peak": round(tf / peak, 4),
                       "peak_tflops": peak, "eager_ms_per_step": round(ms_eager, 4),
                       "eager_shard_fwd_us": round(shard_us, 2),
                       "eager_shard_fwd_median_us": round(shard_st["median"], 2),
                       "eager_shard_fwd_p10_us": round(shard_st["p10"], 2),
                       "eager_shard_fwd_p90_us": round(shard_st["p90"], 2),
                       "eager_shard_fwd_calls": shard_st["calls"]}
        keep[w.name] = (w, host, y)
        log(f"[bench] {w.name}: {ms:.3f} ms/step as a graph ({tf:.1f} TFLOP/s, all ranks + sum); "
            f"eager {ms_eager:.3f} ms")
    return res, keep


def cpu_check_configs(results: dict, kept: dict, rows_n: int = 1024) -> None:
    """The oracle on a seeded sample of token rows of each smaller workload, against the
    GPU's reduced output y (normwise max error, and the oracle's time for the sample)."""
    import numpy as np

    from megatron_tensor_transformer_gemm_amd import inputs as I
    from oracle import tp_oracle as O

    for name, (w, host, y) in kept.items():
        g = np.random.default_rng(4321 + w.cid)
        rows = np.unique(np.concatenate([[0, w.T - 1], g.choice(w.T, size=min(rows_n, w.T), replace=False)]))
        x = I.as_f64(host["x"], w.dtype)[rows]
        w1, w2 = I.as_f64(host["w1"], w.dtype), I.as_f64(host["w2"], w.dtype)
        w3 = I.as_f64(host["w3"], w.dtype) if "w3" in host else None
        t0 = time.perf_counter()
        ref = O.partial_sum([O.ffn_shard(x, w1, w3, w2, w.T_p, t, w.act)[1] for t in range(w.T_p)])
        secs = time.perf_counter() - t0
        got = y.float().cpu().numpy().astype(np.float64)[rows]
        err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        tol = 1e-5 if w.dtype == I.F32 else 2e-2
        results[name].update({"max_err": err, "tolerance": tol, "pass": err <= tol,
                              "oracle_rows": int(len(rows)), "oracle_seconds": round(secs, 2)})
        if err > tol:
            log(f"[bench] PARITY FAILURE: {name} max_err {err:.3e} > {tol}")


def cpu_baseline(host, w, Y, A, rows_n: int, repeats: int = 3) -> dict:
    """Time the float64 oracle on a sample of token rows (all ranks, both sublayers; median
    of `repeats` passes) and compare the GPU's reduced outputs at those rows."""
    import numpy as np

    from megatron_tensor_transformer_gemm_amd import inputs as I
    from oracle import tp_oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    T, d, T_p = w.T, w.d, w.T_p
    n = w.d_ff // T_p
    kdim = w.n_heads // T_p * w.head_dim
    g = np.random.default_rng(1234)
    rows = np.unique(np.concatenate([[0, T - 1], g.choice(T, size=rows_n - 2, replace=False)]))
    R = len(rows)
    log(f"[bench] CPU oracle on {R} token rows, {cores} BLAS threads")
    # decode the bf16 inputs once (exact values); the oracle widens its slices to float64
    xs = I.as_f64(host["x"][rows], w.dtype)
    os_ = I.as_f64(host["o"][rows], w.dtype)
    w1, w3, w2, wo = (I.bf16_to_f32(host[k]) for k in ("w1", "w3", "w2", "wo"))

    def oracle_pass():
        y_parts, a_parts = [], []
        for t in range(T_p):
            _, y_t = O.ffn_shard(xs, w1, w3, w2, T_p, t, w.act)
            y_parts.append(y_t)
            a_parts.append(O.attn_outproj_shard(os_[:, t * kdim:(t + 1) * kdim], wo, w.n_heads,
                                                w.n_kv_heads, w.head_dim, T_p, t))
        return O.partial_sum(y_parts), O.partial_sum(a_parts)

    runs = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        y_ref, a_ref = oracle_pass()
        runs.append(time.perf_counter() - t0)
        log(f"[bench] oracle pass {len(runs)}/{repeats}: {runs[-1]:.1f} s")
    cpu_s = sorted(runs)[len(runs) // 2]
    flops = T_p * R * (2.0 * d * n * 3 + 2.0 * kdim * d)
    yg = Y[rows].float().cpu().numpy()
    ag = A[rows].float().cpu().numpy()
    e_y = O.normwise_max_rel_err(yg, y_ref)
    e_a = O.normwise_max_rel_err(ag, a_ref)
    log(f"[bench] oracle {cpu_s:.1f} s; max err ffn {e_y:.3e} attn {e_a:.3e}")
    if not (e_y <= TOL and e_a <= TOL):
        log(f"[bench] PARITY FAILURE: GPU results differ from the oracle beyond {TOL}")
    return {
        "cpu_baseline": {"value": round(flops / cpu_s / 1e12, 4), "unit": "TFLOP/s", "cores": cores,
                         "kind": "oracle", "seconds": round(cpu_s, 2),
                         "timing": f"median of {len(runs)} passes",
                         "pass_seconds": [round(r, 2) for r in runs],
                         "cores_meaning": "BLAS threads the oracle's matrix products ran on",
                         **host_cpu_info(),
                         "sample": f"{R} of {T} token rows (seeded, incl. first and last); all "
                                   f"{T_p} ranks' SwiGLU FFN shards and attention out-projection "
                                   f"shards plus both partial sums, float64 NumPy"},
        "max_err": {"ffn_sum": e_y, "attn_outproj_sum": e_a, "rows_checked": R,
                    "tolerance": TOL, "pass": bool(e_y <= TOL and e_a <= TOL)},
    }


if __name__ == "__main__":
    sys.exit(main())
