"""Benchmark: head-major non-causal attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]

One step is one ``vattn_forward`` over the whole workload (every head, every
query row) on inputs already resident in HBM.  The K timed steps run as R
replays of one captured HIP graph of K/R launches (``--no-graph``: plain
launches), each replay between two HIP events on the launch stream: the
value is K steps over the whole timed region, and the per-replay times give
the median / p10 / p90 per step.  Prints one JSON line with the attention
throughput 4*H*N^2*d / time, the roofline of the kernel (the dense f16
matrix-core peak, or HBM bandwidth for workloads below the ridge), and the
float64 CPU oracle timed on a bounded sample of the same workload on every
core of the process's affinity mask.

Rotary workloads build their (cos, sin) table once, before timing (it
depends on the positions only, like a weight); a step is then one
``vattn_forward_rope``, which rotates Q and K inside the kernel.
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

METRIC = "attention TFLOP/s (4·H·N²·d) + fraction of MFMA peak, 1 MI355X"
PEAK_F16_TFLOPS = 2516.6   # MI355X dense f16/bf16 matrix peak (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SOURCES = ("non_causal_flash_amd/csrc/attention_fwd.hpp",
                  "non_causal_flash_amd/csrc/vattn.hip")
RIDGE_FLOP_PER_BYTE = PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # ~315


def replay_plan(steps: int, max_replays: int = 10, min_per_graph: int = 10):
    """(replays, launches per graph) with replays * launches == steps.

    Each graph holds at least min_per_graph launches where the step count
    allows it (a graph replay costs tens of microseconds of launch gap, which
    a graph of two 6-20 us launches would put into every step), and among
    those plans the one with the most replays up to max_replays (the per-replay
    times give the spread).  Fewer steps than min_per_graph: one graph of all."""
    steps = max(1, int(steps))
    for r in range(min(max_replays, steps), 0, -1):
        if steps % r == 0 and steps // r >= min(min_per_graph, steps):
            return r, steps // r
    return 1, steps


def roofline_bound(flops: float, algorithmic_bytes: float) -> str:
    """"mfma" when the workload's arithmetic intensity lies above the ridge
    point of the dense f16 peak and HBM bandwidth, "hbm" below it."""
    return "mfma" if flops / algorithmic_bytes >= RIDGE_FLOP_PER_BYTE else "hbm"


def percentile(xs, p: float) -> float:
    """Linear-interpolation percentile of a non-empty sequence."""
    ys = sorted(xs)
    if len(ys) == 1:
        return float(ys[0])
    pos = (len(ys) - 1) * p / 100.0
    lo = int(pos)
    hi = min(lo + 1, len(ys) - 1)
    return float(ys[lo] + (ys[hi] - ys[lo]) * (pos - lo))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "attention_fwd_%s_traffic.txt" % workload_name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_counters(workload_name: str, precision: str):
    """Matrix-core and vector-ALU figures of the attention kernel from the
    committed rocprofv3 counter summary (profiles/attention_fwd_<workload>_mfma.txt,
    one block of lines per precision), or None when there is none for this
    precision or the kernel source changed since it was taken.

    mfma_busy_pct: rocprofv3's MfmaUtil, matrix-core busy cycles over
    GPU-active cycles times the SIMD count; valu_busy_pct: its VALUBusy;
    mfma_f16_flops_per_launch: MfmaFlopsF16, the f16 MFMA work the hardware
    executed (the AUTO/SPLIT corrections and the zero padding of head_dim < 64
    included), next to the algorithmic 4*H*N^2*d."""
    path = os.path.join(ROOT, "profiles", "attention_fwd_%s_mfma.txt" % workload_name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    out = {}
    for key in ("mfma_busy_pct", "valu_busy_pct", "mfma_valu_coexec_pct",
                "mfma_f16_flops_per_launch", "mfma_f16_flops_over_algorithmic"):
        val = fields.get("%s.%s" % (precision, key))
        if val is None:
            return None
        out[key] = float(val)
    out["source"] = os.path.relpath(path, ROOT)
    return out


def oracle_path(q, k, v, w, n_threads: int = 0, rows=None):
    """The whole path in the float64 oracle: rotary transform of Q and K (for
    the rotary workloads), then attention (all rows, or the listed rows)."""
    import oracle
    if w.rope_dims:
        q = oracle.rope_neox_f64(q, w.rope_dims, w.rope_base)
        k = oracle.rope_neox_f64(k, w.rope_dims, w.rope_base)
    if rows is None:
        return oracle.attention_f64(q, k, v, n_threads=n_threads)
    return oracle.attention_rows_f64(q, k, v, rows, n_threads=n_threads)


def cpu_baseline(q, k, v, w, target_s: float):
    """The float64 oracle, untuned, on the first heads of the workload, with
    one OpenMP thread per core of the process's affinity mask; also the
    single-thread time of the two small workloads (whole tensors).  Returns
    the record and the oracle output of the heads it computed."""
    import workloads
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle_path(q[:1], k[:1], v[:1], w, n_threads=cores)
    t1 = time.perf_counter() - t0
    heads = max(1, min(w.n_heads, int(round(target_s / max(t1, 1e-3)))))
    t0 = time.perf_counter()
    ref = oracle_path(q[:heads], k[:heads], v[:heads], w, n_threads=cores)
    dt = time.perf_counter() - t0
    flops = 4.0 * heads * w.n_patches ** 2 * w.head_dim
    single = {}
    for wid in (1, 2):
        sw = workloads.WORKLOADS[wid]
        sq, sk, sv = workloads.make_inputs(wid)
        best = None
        for _ in range(3):
            t0 = time.perf_counter()
            oracle_path(sq, sk, sv, sw, n_threads=1)
            best = min(best or 1e30, time.perf_counter() - t0)
        single[sw.name] = {"seconds": round(best, 5),
                           "gflops": round(sw.flops / best / 1e9, 3)}
    record = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
              "kind": "oracle", "cpu_model": cpu_model(),
              "sample": "first %d of %d heads of %s, every row (%.1f s, float64, %d threads)"
                        % (heads, w.n_heads, w.name, dt, cores),
              "single_thread_best_of_3": single}
    return record, heads, ref


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--precision", default="auto", choices=["auto", "fast", "split"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (0 disables it)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time plain launches instead of one captured HIP graph")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (heads are "
              "independent, so several GPUs would each run the kernel on their own "
              "share of the heads).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import non_causal_flash_amd as vattn
    import workloads

    w = workloads.WORKLOADS[args.workload]
    q, k, v = workloads.make_inputs(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # Device tensors in the workload's storage order, seen as [H, N, d].
    dq, dk, dv = (torch.from_numpy(workloads.to_layout(x, w.layout)).to(dev) for x in (q, k, v))
    out = torch.empty_like(dq)
    if w.layout == "patch":
        dq, dk, dv, out = (t.transpose(0, 1) for t in (dq, dk, dv, out))
    # Everything from here on runs on one non-default stream (default
    # priority), the inputs' host-to-device copies finished first.
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)
    table = vattn.rope_table(w.n_patches, w.rope_dims, w.rope_base) if w.rope_dims else None

    def step():
        vattn.forward(dq, dk, dv, out=out, precision=args.precision, rope=table)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The K timed steps are issued as R replays of one HIP graph of K/R
    # kernel launches (captured once), so that launches of 10-30 us are not
    # paced by the Python call path; --no-graph times plain launches.  HIP
    # events between the replays, on the launch stream, give per-replay
    # times; the timed region is bracketed by synchronisations.
    replays, per_graph = replay_plan(args.steps)
    graph, launch = None, "eager launches"
    if args.graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(per_graph):
                    step()
            graph.replay()  # untimed first replay
            torch.cuda.synchronize()
            launch = ("%d replays of one HIP graph of %d launches, one non-default stream"
                      % (replays, per_graph))
        except RuntimeError as e:  # fall back to plain launches, and say so
            graph, launch = None, "eager launches (graph capture failed: %s)" % str(e)[:80]
            torch.cuda.synchronize()

    events = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    torch.cuda.synchronize()
    events[0].record(stream)
    for r in range(replays):
        if graph is not None:
            graph.replay()
        else:
            for _ in range(per_graph):
                step()
        events[r + 1].record(stream)
    torch.cuda.synchronize()
    ms = events[0].elapsed_time(events[-1]) / args.steps
    per_step = [events[r].elapsed_time(events[r + 1]) / per_graph for r in range(replays)]

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    # spot parity on sampled rows of every head (not timed)
    host_out = out.contiguous().cpu().numpy().astype(np.float64)
    rows = workloads.sample_rows(w.n_heads, w.n_patches, per_head=2)
    got = host_out.reshape(-1, w.head_dim)[rows]
    ref = oracle_path(q, k, v, w, rows=rows)
    diff = got - ref
    parity = {"rows": int(rows.size), "max_abs": float(np.max(np.abs(diff))),
              "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(ref))}

    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9
    traffic = read_traffic(w.name)
    bound = roofline_bound(w.flops, w.algorithmic_bytes)
    if bound == "mfma":
        roofline = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_F16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / PEAK_F16_TFLOPS, 4),
                    "traffic": traffic}
    else:
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "mfma_frac": round(tflops / PEAK_F16_TFLOPS, 4)}
    record = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_spread": {"replays": replays, "launches_per_replay": per_graph,
                               "median": round(percentile(per_step, 50), 5),
                               "p10": round(percentile(per_step, 10), 5),
                               "p90": round(percentile(per_step, 90), 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "n_heads": w.n_heads, "n_patches": w.n_patches,
                   "head_dim": w.head_dim, "precision": args.precision,
                   "rope": ("NeoX rope_dims %d base %g, table built once" % (w.rope_dims, w.rope_base))
                           if w.rope_dims else None,
                   "io": "%s %s resident in HBM" % (w.dtype, "[N][H][d]" if w.layout == "patch" else "[H][N][d]"),
                   "launch": launch},
        "roofline": roofline,
        "hbm_gbs_algorithmic": round(gbs, 1),
        "counters": read_counters(w.name, args.precision),
        "parity_sample": parity,
    }
    if args.cpu_seconds > 0:
        record["cpu_baseline"], heads, ref_heads = cpu_baseline(q, k, v, w, args.cpu_seconds)
        # the baseline's heads, compared in full
        diff = host_out[:heads] - ref_heads
        record["parity_heads"] = {"heads": heads, "elements": int(diff.size),
                                  "max_abs": float(np.max(np.abs(diff))),
                                  "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(ref_heads))}
    else:
        record["cpu_baseline"] = None
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
