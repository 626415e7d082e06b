"""Benchmark: GDN tree verify + commit on one MI355X.

One step = the whole hot path for one batch of draft trees: the accepted
branch of the previous step's trees is committed into the state and the new
trees are verified from the committed state, in one gdn_tree_commit_verify
launch (the commit is the one the verify method defers to the next
iteration).  Workload: one GDN layer, batch 16, 32 heads, d_k = d_v = 128,
64-node trees grown by width-8 best-first expansion (depth <= 12), bf16
q/k/v, fp32 gates and state; seeded synthetic inputs (gdn_synth), no model
weights.

R independent input sets (default 16, ~1.2 GB in total plus pseudo-value
buffers) are resident in HBM before timing and are used round-robin, so the
256 MiB Infinity Cache cannot serve repeated reads.  Step i works on set
i mod R.  Two forms of the step are timed:
  * commit solving (HEADLINE_STEP "solving"): set i's state is advanced
    along the accepted path of set i - 1's tree (its tensors), the commit
    solving for the pseudo-values itself, then set i's tree is verified;
  * pseudo-values carried ("carried", fp32; "carried16", fp16): set i's
    state is advanced along its own tree's accepted path from the
    pseudo-values its previous step wrote from that same state (no solve),
    then its tree is verified again, writing fresh pseudo-values.

Timing: W untimed warmup steps, a clock-settle phase (≥ 30 ms of GPU work on
the verify kernel, so the headline kernel's own dispatches are essentially
its timed ones), then for each form `--regions` (default 5) timed regions of
exactly K steps each, every region bracketed by a device synchronisation and
timed by HIP events on the launch stream (the GPU is kept busy by R untimed
launches queued ahead of the start event, so no launch latency enters).
The reported time is the median region's mean launch time.  Launches are
prepared once (binding Launch objects), so the host enqueues faster than the
GPU drains.

Also timed, each as its own median of regions: the same step as two
launches (gdn_tree_verify then gdn_tree_commit), verify alone and commit
alone; the batch-1 / 32-node layer (latency, each launch replayed from a
captured HIP graph so no host time enters); the 48-layer stack (batch 32,
one fused launch per layer per step); the integer kernels (acceptance walk,
path extraction, tree construction); the tree-size-126 comparison of the
tree verify against single-branch recurrent verification; verify and commit
on the batch-64, 128-node workload.

Prints one JSON line.  `roofline` is for the headline kernel: algorithmic
bytes per launch / its median launch time.  `traffic` is read from the
committed rocprofv3 counter summary when it was taken on the current kernel
source, else null.  `cpu_baseline` times the fp64 oracle (test
infrastructure) on the host cores on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN tree-verify nodes/sec (B=64 tree, batch 16, 32 heads); achieved HBM GB/s"
HBM_PEAK_GBPS = 8000.0
WORKLOAD_INDEX = 2
# the form of the step reported as the headline value (see the docstring)
HEADLINE_STEP = "solving"
# arithmetic of the verify path: bf16 operands feed the MFMA contractions with
# fp32 accumulation; everything else is fp32
KERNEL_DTYPE = "bf16"
TRAFFIC_FILES = {
    "solving": os.path.join(ROOT, "profiles",
                            "commit_verify_solving_b16_n64_h32_d128_traffic.txt"),
}
TRAFFIC_SOURCES = ("commit_verify_mfma.hip", "path_commit.hpp", "tree_verify.hpp",
                   "mfma_tile.hpp", "device_common.hpp")
MAX_PATH = 13            # deepest path of the depth <= 12 trees, plus one
# fp32 matrix peak of the chip (dense), for the all-fp32 verify leg
FP32_MFMA_PEAK_TFLOPS = 157.3
# 32x32x2 fp32 MFMA instructions the all-fp32 verify issues per (sequence,
# head) at 64 nodes: 3 Gram blocks x (Q, K) x 64 k-steps, 4 waves x 256 for
# Q S0 and K S0, 4 waves x 96 for the block solve; 4096 flops each
F32_MFMA_PER_PAIR = 3 * 2 * 64 + 4 * 256 + 4 * 96
GEN_WORKERS = 16         # host processes drawing the synthetic inputs


def verify_bytes(batch, n, H, dk, dv, elem=2):
    """algorithmic HBM bytes of one verify: S0 read once, q/k/v/alpha/beta/parent
    read once, fp32 out written once"""
    per_bh = 4 * dk * dv + n * (2 * dk + dv) * elem + 2 * n * 4 + n * dv * 4
    return batch * H * per_bh + batch * n * 4


def commit_bytes(batch, H, dk, dv, path_lens, elem=2):
    """state read + written once, plus k, v, alpha, beta of every path node and
    the path itself"""
    m = float(sum(path_lens))
    return (batch * H * 2 * 4 * dk * dv + m * H * ((dk + dv) * elem + 8)
            + m * 4 + batch * 4)


def fused_bytes(batch, n, H, dk, dv, path_lens):
    """one commit + verify launch: the state read once and written once, the
    new tree's q/k/v/gates/parents read once, out written once, the path
    nodes' k/v/gates and the path read once"""
    return (verify_bytes(batch, n, H, dk, dv) + commit_bytes(batch, H, dk, dv, path_lens)
            - batch * H * 4 * dk * dv)


FP32_VECTOR_PEAK = 157.3e12   # MI355X fp32 vector FLOP/s (published)


def branch_node_steps(parent):
    """Node updates of the single-branch baseline on one tree: every
    root-to-leaf branch runs its whole path, so sum over leaves of depth + 1."""
    import numpy as np
    import gdn_synth as gs
    parent = np.asarray(parent)
    depth = np.zeros(len(parent), np.int64)
    for i, p in enumerate(parent):
        depth[i] = 0 if p < 0 else depth[p] + 1
    return int(sum(depth[j] + 1 for j in gs.leaves(parent)))


def kernel_source_digest():
    """Digest of the fused kernel's code: its sources with // comments and
    blank lines dropped, so that a comment edit does not void a traffic
    measurement but any code change does."""
    p = os.path.join(ROOT, "gated_deltanet_tree_verify_amd", "csrc")
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(p, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic(step):
    """per-launch HBM bytes of the headline kernel from the committed counter
    summary, or None when the fused kernel's source changed since the
    counters were taken"""
    path = TRAFFIC_FILES.get(step)
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
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


# ---------------------------------------------------------------------------
# input generation (host processes, before the GPU is touched)
# ---------------------------------------------------------------------------
def _draw(job):
    """One seeded input set of a workload; keeps the fp32 copies of q/k/v only
    when asked (the oracle's CPU baseline needs them)."""
    import gdn_synth as gs
    kind, a, keep = job
    if kind == "cfg":
        wi, s = a
        ts = gs.make_config(wi, s=s)
    elif kind == "layer":
        ts = gs.make_config(4, layer=a)
    elif kind == "f32":
        # the 64-node workload's tree shapes with all-fp32 q/k/v
        import numpy as np
        ts = gs.make_set(gs.make_trees(2, np.random.default_rng(1000 + a)), 32, 128, 128,
                         "fp32", seed=1000 + a)
        return ts
    else:
        ts = gs.make_tree126(a)
    if not keep:
        ts.q = ts.k = ts.v = None
    return ts


def draw_all(jobs, workers):
    """every job drawn by a pool of fresh interpreter processes (a worker
    that dies raises here instead of being replaced)"""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    nw = max(1, min(workers, len(os.sched_getaffinity(0)), len(jobs)))
    if nw == 1:
        return [_draw(j) for j in jobs]
    with ProcessPoolExecutor(nw, mp_context=mp.get_context("spawn")) as pool:
        return list(pool.map(_draw, jobs))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--regions", type=int, default=5, help="timed regions per measurement")
    ap.add_argument("--sets", type=int, default=16, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the tree-size-126 tree vs single-branch comparison and the "
                         "batch-64 / 128-node side measurement")
    ap.add_argument("--no-stack", action="store_true", help="skip the 48-layer stack")
    ap.add_argument("--no-latency", action="store_true", help="skip the batch-1 latency leg")
    ap.add_argument("--no-fp32", action="store_true",
                    help="skip the all-fp32 leg (64-node workload with fp32 q/k/v)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "every (sequence, head) pair is independent, so a multi-GPU run would shard "
              "sequences or heads with no exchange step, but none is launched here.",
              file=sys.stderr)
        sys.exit(2)
    K, NREG = args.steps, max(1, args.regions)
    log = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))

    import numpy as np
    import gdn_synth as gs

    # ---- every input set, drawn on the host before the GPU is touched
    t0 = time.time()
    jobs = [("cfg", (WORKLOAD_INDEX, s), s == 0) for s in range(args.sets)]
    if not args.no_latency:
        jobs.append(("cfg", (1, 0), False))
    if not args.no_stack:
        jobs += [("layer", l, False) for l in range(gs.WORKLOADS[4].layers)]
    if not args.no_compare:
        jobs += [("t126", s, False) for s in range(8)]
        jobs += [("cfg", (3, s), False) for s in range(2)]
    if not args.no_fp32:
        jobs += [("f32", s, True) for s in range(2)]
    drawn = draw_all(jobs, GEN_WORKERS)
    pick = lambda kind, a: [ts for (k_, a_, _), ts in zip(jobs, drawn) if k_ == kind and
                            (a is None or a_ == a or (isinstance(a_, tuple) and a_[0] == a))]
    main_host = pick("cfg", WORKLOAD_INDEX)
    log(f"drew {len(jobs)} input sets on {min(GEN_WORKERS, len(os.sched_getaffinity(0)))} "
        f"host processes in {time.time() - t0:.1f}s")

    import torch
    import gated_deltanet_tree_verify_amd as g

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    g.load()
    w = gs.WORKLOADS[WORKLOAD_INDEX]
    batch, n, H, dk, dv = w.batch, w.n, w.H, w.d_k, w.d_v
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    def upload(ts, max_path):
        path, plen = ts.paths(max_path=max_path)
        return dict(q=dev(ts.q_bits.view(np.int16)).view(torch.bfloat16),
                    k=dev(ts.k_bits.view(np.int16)).view(torch.bfloat16),
                    v=dev(ts.v_bits.view(np.int16)).view(torch.bfloat16),
                    alpha=dev(ts.alpha), beta=dev(ts.beta), parent=dev(ts.parent),
                    S=dev(ts.S0), path=dev(path), plen=dev(plen), plen_host=plen)

    def regions(body, nsteps, preroll, nreg=NREG):
        """median over nreg regions of the mean time (ms) of nsteps calls of
        body(i); preroll untimed calls keep the GPU busy ahead of the start"""
        per, host = [], []
        i = 0
        for _ in range(nreg):
            torch.cuda.synchronize()
            for _ in range(preroll):
                body(i)
                i += 1
            e0, e1 = ev(), ev()
            e0.record(stream)
            h0 = time.perf_counter()
            for _ in range(nsteps):
                body(i)
                i += 1
            host.append((time.perf_counter() - h0) / nsteps)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / nsteps)
        return statistics.median(per), per, statistics.median(host)

    # ---- the batch-16 / 64-node layer, R rotating sets
    sets = [upload(ts, MAX_PATH) for ts in main_host]
    for d in sets:
        d["out"] = torch.empty((batch, n, H, dv), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    resident = sum(t.numel() * t.element_size() for d in sets for t in d.values()
                   if isinstance(t, torch.Tensor))
    log(f"{len(sets)} sets of {w.name} resident ({resident / 2**30:.2f} GiB)")
    R = len(sets)
    own = lambda d: (d["k"], d["v"], d["alpha"], d["beta"], d["parent"])
    zero_plen = torch.zeros(batch, dtype=torch.int32, device="cuda")
    carried, carried16, seed16, solving, ver, com = [], [], [], [], [], []
    for i, d in enumerate(sets):
        for key, udt in (("u", torch.float32), ("u16", torch.float16)):
            d[key] = [torch.empty((batch, n, H, dv), dtype=udt, device="cuda") for _ in range(2)]
        # first call on this state: no commit, pseudo-values into u[0]
        g.commit_verify(d["S"], d["path"], zero_plen, own(d), d["q"], d["k"], d["v"],
                        d["alpha"], d["beta"], d["parent"], out=d["out"], u_out=d["u"][0],
                        stream=stream)
        fv = lambda d, key, par, up=True: g.commit_verify(
            d["S"], d["path"], d["plen"], own(d), d["q"], d["k"], d["v"], d["alpha"],
            d["beta"], d["parent"], out=d["out"], u_prev=d[key][par] if up else None,
            u_out=d[key][1 - par], stream=stream, prepare=True)
        carried.append([fv(d, "u", par) for par in range(2)])
        carried16.append([fv(d, "u16", par) for par in range(2)])
        seed16.append(g.commit_verify(d["S"], d["path"], zero_plen, own(d), d["q"], d["k"],
                                      d["v"], d["alpha"], d["beta"], d["parent"], out=d["out"],
                                      u_out=d["u16"][0], stream=stream, prepare=True))
        p = sets[(i - 1) % R]
        solving.append(g.commit_verify(d["S"], p["path"], p["plen"], own(p), d["q"], d["k"],
                                       d["v"], d["alpha"], d["beta"], d["parent"], out=d["out"],
                                       stream=stream, prepare=True))
        ver.append(g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"],
                            out=d["out"], stream=stream, prepare=True))
        com.append(g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"], d["alpha"], d["beta"],
                            d["parent"], stream=stream, prepare=True))
    visits = {"u": [0] * R, "u16": [0] * R}

    def carried_step(i, key="u", calls=None):
        j = i % R
        (calls or carried)[j][visits[key][j] & 1]()
        visits[key][j] += 1

    steps = {
        "carried": carried_step,
        "carried16": lambda i: carried_step(i, "u16", carried16),
        "solving": lambda i: solving[i % R](),
    }
    head = steps[HEADLINE_STEP]
    for i in range(args.warmup):
        head(i)
    torch.cuda.synchronize()
    # Clocks settle only after some milliseconds of sustained load; the
    # settle phase runs the verify kernel, so that the headline kernel's
    # dispatches are its warmup, its prerolls and its timed ones.
    e0, e1 = ev(), ev()
    e0.record(stream)
    settled = 0
    while True:
        for i in range(100):
            ver[i % R]()
        e1.record(stream)
        e1.synchronize()
        settled += 100
        if e0.elapsed_time(e1) >= 30.0 or settled >= 20000:
            break

    res = {}
    res[HEADLINE_STEP] = regions(head, K, R)
    # the fp16 chain starts from a first call on each set's current state
    for i in range(R):
        seed16[i]()
    visits["u16"] = [0] * R
    for name in ("carried", "carried16", "solving"):
        if name not in res:
            if name == "carried":
                # reseed the fp32 chain from the current states
                for j, d in enumerate(sets):
                    g.commit_verify(d["S"], d["path"], zero_plen, own(d), d["q"], d["k"],
                                    d["v"], d["alpha"], d["beta"], d["parent"], out=d["out"],
                                    u_out=d["u"][visits["u"][j] & 1], stream=stream)
            res[name] = regions(steps[name], K, R)
    res["separate"] = regions(lambda i: (ver[i % R](), com[i % R]()), K, R)
    res["verify"] = regions(lambda i: ver[i % R](), K, R)
    res["commit"] = regions(lambda i: com[i % R](), K, R)
    us = {k_: v_[0] * 1e3 for k_, v_ in res.items()}
    log("batch-16 layer, median of %d regions of %d launches: " % (NREG, K) +
        ", ".join(f"{k_} {v_:.2f} us" for k_, v_ in us.items()) +
        f" (host enqueue {res[HEADLINE_STEP][2] * 1e6:.1f} us per launch)")
    log(f"  {HEADLINE_STEP} regions: " + " ".join(f"{x * 1e3:.2f}" for x in res[HEADLINE_STEP][1]))

    nodes = batch * n
    mean_plen = float(np.mean([float(np.sum(d["plen_host"])) for d in sets]))
    vbytes = verify_bytes(batch, n, H, dk, dv)
    cbytes = commit_bytes(batch, H, dk, dv, [mean_plen])
    fbytes = fused_bytes(batch, n, H, dk, dv, [mean_plen])
    ms_step = res[HEADLINE_STEP][0]
    step_s = ms_step * 1e-3
    achieved = fbytes / step_s / 1e9

    # ---- the step's integer kernels on the same trees
    ts0 = main_host[0]
    draft, vtok = gs.make_accept_tokens(np.random.default_rng(0), ts0.parent, p_match=0.8)
    dpar, ddraft, dvtok = dev(ts0.parent), dev(draft), dev(vtok)
    acc_call = g.accept(dpar, ddraft, dvtok, stream=stream, prepare=True)
    acc_t, _, _ = acc_call()
    path_call = g.path(dpar, acc_t, MAX_PATH, stream=stream, prepare=True)
    clp, ctok, croot = gs.candidate_table(np.random.default_rng(1), batch, n, 8)
    build_call = g.build_tree(dev(clp), dev(ctok), dev(croot), 8, 12, stream=stream,
                              prepare=True)
    small = lambda call: regions(lambda i: call(), 100, 5, 3)[0] * 1e3
    accept_us, path_us, build_us = small(acc_call), small(path_call), small(build_call)
    sets = carried = carried16 = seed16 = solving = ver = com = None
    torch.cuda.empty_cache()

    # ---- batch 1, 32 heads, 32-node tree: latency of each launch, replayed
    # from a captured HIP graph (64 launches per replay, no host time inside)
    lat = None
    if not args.no_latency:
        w1 = gs.WORKLOADS[1]
        ts1 = pick("cfg", 1)[0]
        mp1 = int(ts1.paths()[1].max())
        d = upload(ts1, mp1)
        d["out"] = torch.empty((1, w1.n, w1.H, w1.d_v), dtype=torch.float32, device="cuda")
        d["u"] = [torch.empty((1, w1.n, w1.H, w1.d_v), dtype=torch.float32, device="cuda")
                  for _ in range(2)]
        z1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        g.commit_verify(d["S"], d["path"], z1, own(d), d["q"], d["k"], d["v"], d["alpha"],
                        d["beta"], d["parent"], out=d["out"], u_out=d["u"][0], stream=stream)
        torch.cuda.synchronize()
        S_keep = d["S"].clone()
        kinds = {
            "verify": lambda j: g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                         d["parent"], d["S"], out=d["out"]),
            "commit": lambda j: g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"],
                                         d["alpha"], d["beta"], d["parent"]),
            "fused_solving": lambda j: g.commit_verify(
                d["S"], d["path"], d["plen"], own(d), d["q"], d["k"], d["v"], d["alpha"],
                d["beta"], d["parent"], out=d["out"]),
            "fused_carried": lambda j: g.commit_verify(
                d["S"], d["path"], d["plen"], own(d), d["q"], d["k"], d["v"], d["alpha"],
                d["beta"], d["parent"], out=d["out"], u_prev=d["u"][j & 1],
                u_out=d["u"][1 - (j & 1)]),
        }
        # the same layer cut to its first 8 heads (a quarter of the
        # workgroups): if the latency stays, the chain of dependent stages
        # inside one workgroup sets it, not the number of CUs the launch
        # occupies
        d8 = {k_: (v_[:, :, :8].contiguous() if v_.dim() >= 3 else v_.clone())
              for k_, v_ in d.items() if isinstance(v_, torch.Tensor) and k_ not in ("S", "u")}
        d8["S"] = d["S"][:, :8].contiguous()
        kinds["verify_h8"] = lambda j: g.verify(d8["q"], d8["k"], d8["v"], d8["alpha"],
                                                d8["beta"], d8["parent"], d8["S"],
                                                out=d8["out"])
        lat = {"workload": w1.name, "launches_per_graph": 64}
        for name, call in kinds.items():
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for j in range(2):
                    call(j)
            stream.wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for j in range(64):
                    call(j)
            torch.cuda.synchronize()
            lat[name + "_us"] = regions(lambda i: graph.replay(), 5, 1)[0] * 1e3 / 64
            d["S"].copy_(S_keep)
            del graph
        log("batch-1 layer (graph-replayed launches): " +
            ", ".join(f"{k_[:-3]} {v_:.2f} us" for k_, v_ in lat.items() if k_.endswith("_us")))
        d = None
        torch.cuda.empty_cache()

    # ---- the 48-layer stack: batch 32, one 64-node tree per sequence shared
    # by the layers; a step runs every layer's fused launch in layer order
    stack = None
    if not args.no_stack:
        w4 = gs.WORKLOADS[4]
        layers = pick("layer", None)
        L = len(layers)
        ls = [upload(ts, MAX_PATH) for ts in layers]
        for d in ls:
            d["out"] = torch.empty((w4.batch, w4.n, w4.H, w4.d_v), dtype=torch.float32,
                                   device="cuda")
        layers = None
        zero32 = torch.zeros(w4.batch, dtype=torch.int32, device="cuda")
        if HEADLINE_STEP == "solving":
            calls = [[g.commit_verify(d["S"], d["path"], d["plen"], own(d), d["q"], d["k"],
                                      d["v"], d["alpha"], d["beta"], d["parent"], out=d["out"],
                                      stream=stream, prepare=True)] * 2 for d in ls]
        else:
            calls = []
            for d in ls:
                d["u"] = [torch.empty_like(d["out"]) for _ in range(2)]
                g.commit_verify(d["S"], d["path"], zero32, own(d), d["q"], d["k"], d["v"],
                                d["alpha"], d["beta"], d["parent"], out=d["out"],
                                u_out=d["u"][0], stream=stream)
                calls.append([g.commit_verify(
                    d["S"], d["path"], d["plen"], own(d), d["q"], d["k"], d["v"], d["alpha"],
                    d["beta"], d["parent"], out=d["out"], u_prev=d["u"][par],
                    u_out=d["u"][1 - par], stream=stream, prepare=True) for par in range(2)])
        torch.cuda.synchronize()
        sres = {"par": 0}

        def stack_step(i):
            for c in calls:
                c[sres["par"]]()
            sres["par"] ^= 1

        for i in range(max(1, args.warmup // 4)):
            stack_step(i)
        ms4, per4, _ = regions(stack_step, max(2, K // 4), 1)
        m4 = float(np.mean([float(np.sum(d["plen_host"])) for d in ls]))
        b4 = L * fused_bytes(w4.batch, w4.n, w4.H, w4.d_k, w4.d_v, [m4])
        stack = {"workload": w4.name, "layers": L, "step": HEADLINE_STEP,
                 "ms_per_step": ms4, "nodes_per_s": w4.batch * w4.n / (ms4 * 1e-3),
                 "layer_launch_us": ms4 * 1e3 / L, "algorithmic_bytes_per_step": b4,
                 "hbm_gbps": b4 / (ms4 * 1e-3) / 1e9,
                 "frac": b4 / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "regions_ms": per4, "steps_per_region": max(2, K // 4)}
        log(f"48-layer stack: {ms4:.3f} ms/step ({ms4 * 1e3 / L:.1f} us per layer), "
            f"{stack['hbm_gbps']:.0f} GB/s algorithmic ({stack['frac']:.3f} of 8 TB/s)")
        ls = calls = None
        torch.cuda.empty_cache()

    # ---- tree-size-126 comparison and the batch-64 / 128-node workload
    cmp126 = b64 = None
    if not args.no_compare:
        c_sets = []
        for ts in pick("t126", None):
            d = upload(ts, 17)     # depth <= 16: paths of at most 17 nodes
            # the same accepted paths cut to their first 16 nodes (a path to
            # an ancestor of the accepted leaf), for the decode-step timing
            d["path16"] = d["path"][:, :16].contiguous()
            d["plen16"] = torch.clamp(d["plen"], max=16)
            d["m16"] = float(np.sum(np.minimum(d["plen_host"], 16)))
            d["leaves"] = sum(len(gs.leaves(p)) for p in ts.parent)
            d["steps"] = sum(branch_node_steps(p) for p in ts.parent)
            d["out"] = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
            c_sets.append(d)
        tv126 = [g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"],
                          out=d["out"], stream=stream, prepare=True) for d in c_sets]
        bv126 = [g.branch_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                                 d["S"], out=d["out"], stream=stream, prepare=True)
                 for d in c_sets]
        # the decode step on these trees: set i's state advanced along set
        # i - 1's accepted path, then set i's trees verified: one fused
        # launch, or a commit launch and a verify launch
        fs126 = [g.commit_verify(d["S"], c_sets[i - 1]["path16"], c_sets[i - 1]["plen16"],
                                 own(c_sets[i - 1]), d["q"], d["k"], d["v"], d["alpha"],
                                 d["beta"], d["parent"], out=d["out"], stream=stream, prepare=True)
                 for i, d in enumerate(c_sets)]
        cm126 = [g.commit(d["S"], c_sets[i - 1]["path16"], c_sets[i - 1]["plen16"],
                          *own(c_sets[i - 1]),
                          stream=stream, prepare=True) for i, d in enumerate(c_sets)]
        t_tree = regions(lambda i: tv126[i % 8](), 40, 8)[0] * 1e3
        t_branch = regions(lambda i: bv126[i % 8](), 10, 2, 3)[0] * 1e3
        t_fs126 = regions(lambda i: fs126[i % 8](), 40, 8)[0] * 1e3
        t_sep126 = regions(lambda i: (cm126[i % 8](), tv126[i % 8]()), 40, 8)[0] * 1e3
        w126 = gs.TREE126
        # what the branch baseline computes: per branch node and head,
        # w = S^T k (2 d^2 flops), the update alpha S + (beta k)(v - alpha w)^T
        # (3 d^2) and o = S^T q (2 d^2); on the fp32 vector peak this is a
        # floor for any recurrent branch verify on this chip
        steps126 = float(np.mean([d["steps"] for d in c_sets]))   # per set, all sequences
        branch_flop = steps126 * w126.H * 7 * w126.d_k * w126.d_v
        floor_us = branch_flop / FP32_VECTOR_PEAK * 1e6
        cmp126 = {"workload": w126.name, "tree_verify_us": t_tree, "branch_verify_us": t_branch,
                  "speedup": t_branch / t_tree,
                  "branch_node_steps_per_tree": steps126 / w126.batch,
                  "branch_tflop_per_s": branch_flop / (t_branch * 1e-6) / 1e12,
                  "branch_fp32_floor_us": floor_us,
                  "speedup_vs_branch_floor": floor_us / t_tree,
                  "mean_leaves_per_tree": float(np.mean([d["leaves"] / w126.batch
                                                         for d in c_sets])),
                  "tree_verify_nodes_per_s": w126.batch * w126.n / (t_tree * 1e-6),
                  "tree_verify_hbm_gbps": verify_bytes(w126.batch, w126.n, w126.H, w126.d_k,
                                                       w126.d_v) / (t_tree * 1e-6) / 1e9,
                  "tree_verify_algorithmic_bytes": verify_bytes(w126.batch, w126.n, w126.H,
                                                                w126.d_k, w126.d_v),
                  "decode_step_paths16": {
                      "one_launch_us": t_fs126, "commit_then_verify_us": t_sep126,
                      "algorithmic_bytes": fused_bytes(
                          w126.batch, w126.n, w126.H, w126.d_k, w126.d_v,
                          [float(np.mean([d["m16"] for d in c_sets]))])},
                  "pages_speedup_b200": 7.1}
        log(f"n=126: tree verify {t_tree:.1f} us, branch verify {t_branch:.1f} us, "
            f"speedup {t_branch / t_tree:.2f} (branch at {cmp126['branch_tflop_per_s']:.1f} "
            f"TFLOP/s; its fp32 floor {floor_us:.0f} us, {floor_us / t_tree:.2f}x the tree); "
            f"decode step: fused {t_fs126:.1f} us, two launches {t_sep126:.1f} us")
        c_sets = tv126 = bv126 = fs126 = cm126 = None
        torch.cuda.empty_cache()

        w3 = gs.WORKLOADS[3]
        b_sets = []
        for ts in pick("cfg", 3):
            d = upload(ts, w3.n)
            d["m"] = float(np.sum(d["plen_host"]))
            d["out"] = torch.empty((w3.batch, w3.n, w3.H, w3.d_v), dtype=torch.float32,
                                   device="cuda")
            b_sets.append(d)
        vb = [g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"],
                       out=d["out"], stream=stream, prepare=True) for d in b_sets]
        cb = [g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"], d["alpha"], d["beta"],
                       d["parent"], stream=stream, prepare=True) for d in b_sets]
        # the fused step on this workload: set i's state advanced along set
        # i - 1's accepted paths (the commit solving), then set i's trees
        # verified in one launch, without and with the new pseudo-values
        # out; and the same as a commit launch then a verify launch
        for d in b_sets:
            d["u"] = torch.empty_like(d["out"])
        fb = [g.commit_verify(d["S"], b_sets[(i - 1) % 2]["path"], b_sets[(i - 1) % 2]["plen"],
                              own(b_sets[(i - 1) % 2]), d["q"], d["k"], d["v"], d["alpha"],
                              d["beta"], d["parent"], out=d["out"], stream=stream, prepare=True)
              for i, d in enumerate(b_sets)]
        fbu = [g.commit_verify(d["S"], b_sets[(i - 1) % 2]["path"], b_sets[(i - 1) % 2]["plen"],
                               own(b_sets[(i - 1) % 2]), d["q"], d["k"], d["v"], d["alpha"],
                               d["beta"], d["parent"], out=d["out"], u_out=d["u"],
                               stream=stream, prepare=True)
               for i, d in enumerate(b_sets)]
        cbp = [g.commit(d["S"], b_sets[(i - 1) % 2]["path"], b_sets[(i - 1) % 2]["plen"],
                        *own(b_sets[(i - 1) % 2]), stream=stream, prepare=True)
               for i, d in enumerate(b_sets)]
        t_vb = regions(lambda i: vb[i % 2](), 20, 2)[0] * 1e3
        t_cb = regions(lambda i: cb[i % 2](), 20, 2)[0] * 1e3
        t_fb = regions(lambda i: fb[i % 2](), 20, 2)[0] * 1e3
        t_fbu = regions(lambda i: fbu[i % 2](), 20, 2)[0] * 1e3
        t_sep = regions(lambda i: (cbp[i % 2](), vb[i % 2]()), 20, 2)[0] * 1e3
        vb_bytes = verify_bytes(w3.batch, w3.n, w3.H, w3.d_k, w3.d_v)
        cb_bytes = commit_bytes(w3.batch, w3.H, w3.d_k, w3.d_v,
                                [float(np.mean([d["m"] for d in b_sets]))])
        fb_bytes = vb_bytes + cb_bytes - w3.batch * w3.H * 4 * w3.d_k * w3.d_v
        b64 = {"workload": w3.name, "verify_us": t_vb, "commit_us": t_cb,
               "commit_verify_us": t_fb, "commit_verify_u_out_us": t_fbu,
               "commit_then_verify_us": t_sep,
               "commit_verify_hbm_gbps": fb_bytes / (t_fb * 1e-6) / 1e9,
               "commit_verify_frac": fb_bytes / (t_fb * 1e-6) / 1e9 / HBM_PEAK_GBPS,
               "verify_nodes_per_s": w3.batch * w3.n / (t_vb * 1e-6),
               "verify_hbm_gbps": vb_bytes / (t_vb * 1e-6) / 1e9,
               "verify_frac": vb_bytes / (t_vb * 1e-6) / 1e9 / HBM_PEAK_GBPS,
               "commit_hbm_gbps": cb_bytes / (t_cb * 1e-6) / 1e9,
               "verify_algorithmic_bytes": vb_bytes, "commit_algorithmic_bytes": cb_bytes,
               "commit_verify_algorithmic_bytes": fb_bytes}
        log(f"b64/n128: verify {t_vb:.1f} us ({b64['verify_hbm_gbps']:.0f} GB/s, "
            f"{b64['verify_frac']:.3f}), commit {t_cb:.1f} us ({b64['commit_hbm_gbps']:.0f} GB/s), "
            f"commit_verify {t_fb:.1f} us ({b64['commit_verify_frac']:.3f}; with u_out "
            f"{t_fbu:.1f} us; as two launches {t_sep:.1f} us)")
        b_sets = vb = cb = cbp = fb = fbu = None
        torch.cuda.empty_cache()

    # ---- the same 64-node workload with all-fp32 q/k/v: the verify on the
    #      fp32-MFMA kernel, the commit and the fused call on the generic
    #      kernels (the fused call is a commit launch then that verify)
    f32 = None
    if not args.no_fp32:
        f_sets = []
        for ts in pick("f32", None):
            path, plen = ts.paths(max_path=MAX_PATH)
            d = dict(q=dev(ts.q), k=dev(ts.k), v=dev(ts.v), alpha=dev(ts.alpha),
                     beta=dev(ts.beta), parent=dev(ts.parent), S=dev(ts.S0), path=dev(path),
                     plen=dev(plen), m=float(np.sum(plen)))
            d["out"] = torch.empty((batch, n, H, dv), dtype=torch.float32, device="cuda")
            f_sets.append(d)
        vf = [g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"],
                       out=d["out"], stream=stream, prepare=True) for d in f_sets]
        cf = [g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"], d["alpha"], d["beta"],
                       d["parent"], stream=stream, prepare=True) for d in f_sets]
        ff = [g.commit_verify(d["S"], f_sets[(i - 1) % 2]["path"], f_sets[(i - 1) % 2]["plen"],
                              own(f_sets[(i - 1) % 2]), d["q"], d["k"], d["v"], d["alpha"],
                              d["beta"], d["parent"], out=d["out"], stream=stream, prepare=True)
              for i, d in enumerate(f_sets)]
        t_vf = regions(lambda i: vf[i % 2](), 20, 2)[0] * 1e3
        t_cf = regions(lambda i: cf[i % 2](), 4, 1)[0] * 1e3
        t_ff = regions(lambda i: ff[i % 2](), 4, 1)[0] * 1e3
        vf_bytes = verify_bytes(batch, n, H, dk, dv, elem=4)
        cf_bytes = commit_bytes(batch, H, dk, dv, [np.mean([d["m"] for d in f_sets])], elem=4)
        vf_tflops = batch * H * F32_MFMA_PER_PAIR * 4096 / (t_vf * 1e-6) / 1e12
        f32 = {"workload": w.name + "-fp32", "verify_us": t_vf, "commit_us": t_cf,
               "commit_verify_us": t_ff,
               "verify_nodes_per_s": batch * n / (t_vf * 1e-6),
               "verify_hbm_gbps": vf_bytes / (t_vf * 1e-6) / 1e9,
               "verify_mfma_tflops": vf_tflops,
               "verify_mfma_frac": vf_tflops / FP32_MFMA_PEAK_TFLOPS,
               "commit_hbm_gbps": cf_bytes / (t_cf * 1e-6) / 1e9,
               "verify_algorithmic_bytes": vf_bytes, "commit_algorithmic_bytes": cf_bytes}
        log(f"fp32 b16/n64: verify {t_vf:.1f} us ({vf_tflops:.1f} TFLOP/s on the fp32 matrix "
            f"units, {f32['verify_hbm_gbps']:.0f} GB/s), commit {t_cf:.1f} us, "
            f"commit_verify {t_ff:.1f} us")
        f_sets = vf = cf = ff = None
        torch.cuda.empty_cache()

    # ---- achievable-bandwidth line: a plain 1 GiB device copy
    src = torch.empty(2**28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = regions(lambda i: dst.copy_(src), 5, 1, 3)[0]
    copy_gbps = 2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9
    del src, dst

    result = {
        "metric": METRIC,
        "value": nodes / step_s,
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
                   "d_v": dv, "tree": "width-8 best-first, depth<=12", "rotating_sets": R,
                   "step": {"carried": "commit the accepted path (fp32 pseudo-values carried "
                                       "from the previous verify) + verify the trees, writing "
                                       "their pseudo-values (one launch)",
                            "solving": "commit the previous trees' accepted paths (the commit "
                                       "solving for its pseudo-values) + verify the trees "
                                       "(one launch)"}[HEADLINE_STEP],
                   "timing": f"median of {NREG} regions of {K} launches"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": read_traffic(HEADLINE_STEP),
                     "kernel": "gdn_tree_commit_verify (%s)" % HEADLINE_STEP,
                     "algorithmic_bytes_per_launch": fbytes,
                     "median_launch_us": step_s * 1e6, "target_frac": 0.60,
                     "frac_of_copy": achieved / copy_gbps},
        "region_us": {k_: [x * 1e3 for x in v_[1]] for k_, v_ in res.items()},
        "fused_carried_us": us["carried"],
        "fused_carried_fp16_us": us["carried16"],
        "fused_solving_us": us["solving"],
        "separate_step_us": us["separate"],
        "separate_step_nodes_per_s": nodes / (res["separate"][0] * 1e-3),
        "verify_us": us["verify"],
        "commit_us": us["commit"],
        "verify_nodes_per_s": nodes / (res["verify"][0] * 1e-3),
        "verify_hbm_gbps": vbytes / (res["verify"][0] * 1e-3) / 1e9,
        "commit_hbm_gbps": cbytes / (res["commit"][0] * 1e-3) / 1e9,
        "host_enqueue_us_per_step": res[HEADLINE_STEP][2] * 1e6,
        "copy_gbps": copy_gbps,
        "verify_frac_of_copy": vbytes / (res["verify"][0] * 1e-3) / 1e9 / copy_gbps,
        "tree_build_us": build_us,
        "accept_us": accept_us,
        "path_us": path_us,
        "b1_n32": lat,
        "stack48": stack,
        "tree126_vs_branch": cmp126,
        "b64_n128": b64,
        "fp32_b16_n64": f32,
    }
    if not args.no_cpu_baseline:
        ts = main_host[0]
        path, plen = ts.paths(max_path=MAX_PATH)
        result["cpu_baseline"] = cpu_baseline(ts, path, plen)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
