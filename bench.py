"""Benchmark: GDN tree verify + commit on one MI355X.

One step = gdn_tree_verify over a batch of draft trees followed by
gdn_tree_commit of one accepted branch per sequence (the whole hot path).
Workload: one GDN layer, batch 16, 32 heads, d_k = d_v = 128, 64-node trees
grown by width-8 best-first expansion (depth <= 12), bf16 q/k/v, fp32 gates
and state; seeded synthetic inputs (gdn_synth), no model weights.

R independent input sets (default 16, ~1.2 GB in total) are resident in HBM
before timing and are used round-robin, so the 256 MiB Infinity Cache cannot
serve repeated reads; each commit advances its own set's state in place, the
way a decoding loop would.

Timed regions (HIP events on the launch stream, start and end only, so no
event fence sits between kernels): K whole steps (the headline value), then
K back-to-back verify launches and K back-to-back commit launches over the
same rotating sets (per-kernel means; they include the dispatch gap between
consecutive kernels).

Prints one JSON line.  `roofline` is for the verify kernel: algorithmic
bytes per launch / its mean launch time.  `traffic` is read from the
committed rocprofv3 counter summary when it was taken on the current kernel
source, else null.  `cpu_baseline` times the fp64 oracle (test
infrastructure) on the host cores on the same workload.
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

METRIC = "GDN tree-verify nodes/sec (B=64 tree, batch 16, 32 heads); achieved HBM GB/s"
HBM_PEAK_GBPS = 8000.0
WORKLOAD_INDEX = 2
# arithmetic of the verify path: bf16 operands feed the MFMA contractions with
# fp32 accumulation; everything else is fp32
KERNEL_DTYPE = "bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_b16_n64_h32_d128_traffic.txt")


def verify_bytes(batch, n, H, dk, dv, elem=2):
    """algorithmic HBM bytes of one verify: S0 read once, q/k/v/alpha/beta/parent
    read once, fp32 out written once"""
    per_bh = 4 * dk * dv + n * (2 * dk + dv) * elem + 2 * n * 4 + n * dv * 4
    return batch * H * per_bh + batch * n * 4


def commit_bytes(batch, H, dk, dv, path_lens, elem=2, max_path=None):
    """state read + written once, plus k, v, alpha, beta of every path node and
    the path itself"""
    m = int(sum(path_lens))
    return (batch * H * 2 * 4 * dk * dv + m * H * ((dk + dv) * elem + 8)
            + m * 4 + batch * 4)


def kernel_source_digest():
    p = os.path.join(ROOT, "gated_deltanet_tree_verify_amd", "csrc")
    h = hashlib.sha256()
    for f in ("verify_mfma.hip", "verify_generic.hip", "device_common.hpp"):
        with open(os.path.join(p, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """per-launch HBM bytes from the committed counter summary, or None when
    the verify kernel source changed since the counters were taken"""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_digest") != kernel_source_digest():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(ts, path, plen, budget_s=10.0):
    """the fp64 oracle (memoised walk of the explicit recurrence) on the host
    cores: whole steps (verify + commit) of the same workload, repeated until
    about `budget_s` seconds of CPU time have been spent"""
    import oracle
    threads = len(os.sched_getaffinity(0))
    tv = tc = 0.0
    steps = 0
    used = threads
    while tv + tc < budget_s and steps < 1000:
        t0 = time.perf_counter()
        _, _, used = oracle.verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, ts.S0,
                                   memo=True, nthreads=threads, return_threads=True)
        t1 = time.perf_counter()
        oracle.commit(ts.S0, path, plen, ts.k, ts.v, ts.alpha, ts.beta, ts.parent,
                      nthreads=threads)
        t2 = time.perf_counter()
        tv += t1 - t0
        tc += t2 - t1
        steps += 1
    nodes = ts.parent.shape[0] * ts.parent.shape[1]
    return {"value": steps * nodes / (tv + tc), "unit": "nodes/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"{steps} full steps of the same workload ({ts.parent.shape[0]} sequences "
                      f"x {ts.q.shape[2]} heads x {ts.parent.shape[1]} nodes, fp64 verify + "
                      f"commit), {tv + tc:.1f} s",
            "verify_s_per_step": tv / steps, "commit_s_per_step": tc / steps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=16, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "every (sequence, head) pair is independent, so a multi-GPU run would shard "
              "sequences or heads with no exchange step, but none is launched here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_tree_verify_amd as g
    import gdn_synth as gs

    log = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    g.load()
    w = gs.CONFIGS[WORKLOAD_INDEX]
    batch, n, H, dk, dv = w.batch, w.n, w.H, w.d_k, w.d_v
    stream = torch.cuda.current_stream()

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    sets, host0 = [], None
    max_path = 13
    t0 = time.time()
    for s in range(args.sets):
        ts = gs.make_config(WORKLOAD_INDEX, s=s)
        path, plen = ts.paths(max_path=max_path)
        if s == 0:
            host0 = (ts, path, plen)
        d = dict(q=dev(ts.q_bits.view(np.int16)).view(torch.bfloat16),
                 k=dev(ts.k_bits.view(np.int16)).view(torch.bfloat16),
                 v=dev(ts.v_bits.view(np.int16)).view(torch.bfloat16),
                 alpha=dev(ts.alpha), beta=dev(ts.beta), parent=dev(ts.parent), S=dev(ts.S0),
                 path=dev(path), plen=dev(plen), plen_host=plen)
        d["out"] = torch.empty((batch, n, H, dv), dtype=torch.float32, device="cuda")
        sets.append(d)
    torch.cuda.synchronize()
    resident = sum(t.numel() * t.element_size() for d in sets for t in d.values()
                   if isinstance(t, torch.Tensor))
    log(f"generated {args.sets} sets ({resident / 2**30:.2f} GiB resident) in {time.time() - t0:.1f}s")

    def step(d):
        g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"], out=d["out"],
                 stream=stream)
        g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                 stream=stream)

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    K = args.steps

    def timed(body):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K):
            body(sets[i % len(sets)])
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    def verify_only(d):
        g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"], out=d["out"],
                 stream=stream)

    def commit_only(d):
        g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                 stream=stream)

    ms_step = timed(step)
    ver_ms = timed(verify_only)
    com_ms = timed(commit_only)
    nodes = batch * n
    vbytes = verify_bytes(batch, n, H, dk, dv)
    mean_plen = float(np.mean([float(np.sum(d["plen_host"])) for d in sets]))
    cbytes = commit_bytes(batch, H, dk, dv, [mean_plen])
    v_mean_s = ver_ms * 1e-3
    c_mean_s = com_ms * 1e-3
    achieved = vbytes / v_mean_s / 1e9
    traffic = read_traffic()

    # achievable-bandwidth line: a plain 1 GiB device copy
    src = torch.empty(2**28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    result = {
        "metric": METRIC,
        "value": nodes / (ms_step * 1e-3),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": KERNEL_DTYPE,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": batch, "tree_nodes": n, "heads": H, "d_k": dk,
                   "d_v": dv, "tree": "width-8 best-first, depth<=12", "rotating_sets": args.sets,
                   "step": "verify + commit"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "gdn_tree_verify", "algorithmic_bytes_per_launch": vbytes,
                     "mean_launch_us": v_mean_s * 1e6},
        "verify_us": v_mean_s * 1e6,
        "commit_us": c_mean_s * 1e6,
        "verify_nodes_per_s": nodes / v_mean_s,
        "step_hbm_gbps": (vbytes + cbytes) / (ms_step * 1e-3) / 1e9,
        "commit_hbm_gbps": cbytes / c_mean_s / 1e9,
        "copy_gbps": copy_gbps,
    }
    if not args.no_cpu_baseline:
        ts, path, plen = host0
        result["cpu_baseline"] = cpu_baseline(ts, path, plen)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
