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
i mod R: its state is advanced along the accepted path of its own tree,
from the pseudo-values its previous step wrote from that same state (the
commit then needs no solve), and its tree is verified again, writing fresh
pseudo-values; a first call per set (no commit) seeds them.

Timed regions (HIP events on the launch stream, start and end only, so no
event fence sits between kernels), K launches each after 2R untimed ones:
the fused step (the headline value), the same with fp16 pseudo-values, the
fused step with the commit solving for the pseudo-values itself (set i - 1's
path), the same step as two launches (gdn_tree_verify then gdn_tree_commit),
verify alone and commit alone.  Launches are prepared
once (binding Launch objects), so the host enqueues faster than the GPU
drains and the events time the GPU.

Side measurements (not the headline): the integer kernels of the step
(acceptance walk, path extraction, tree construction); the tree-size-126
comparison of the tree verify against single-branch recurrent
verification; verify and commit on the batch-64, 128-node workload.

Prints one JSON line.  `roofline` is for the fused kernel: algorithmic bytes
per launch / its mean launch time.  `traffic` is read from the committed
rocprofv3 counter summary when it was taken on the current kernel source,
else null.  `cpu_baseline` times the fp64 oracle (test infrastructure) on
the host cores on the same workload.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "commit_verify_b16_n64_h32_d128_traffic.txt")
TRAFFIC_SOURCES = ("commit_verify_mfma.hip", "path_commit.hpp", "tree_verify.hpp",
                   "mfma_tile.hpp", "device_common.hpp")


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


def read_traffic():
    """per-launch HBM bytes from the committed counter summary, or None when
    the fused kernel's source changed since the counters were taken"""
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
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the tree-size-126 tree vs single-branch comparison and the "
                         "batch-64 / 128-node side measurement")
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
    w = gs.WORKLOADS[WORKLOAD_INDEX]
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

    R = len(sets)
    # The step (fused_u): set i's state is advanced along its own tree's
    # accepted path from the pseudo-values its previous verify wrote from that
    # same state, then the tree is verified again and writes fresh
    # pseudo-values (two buffers per set, alternating).  fused_solve,
    # reported beside it: set i's state is advanced along set i - 1's path
    # with the commit solving for the pseudo-values itself.
    fused_u, fused_u16, seed_u16, fused_solve, ver, com = [], [], [], [], [], []
    for i, d in enumerate(sets):
        own = (d["k"], d["v"], d["alpha"], d["beta"], d["parent"])
        for key, udt in (("u", torch.float32), ("u16", torch.float16)):
            d[key] = [torch.empty((batch, n, H, dv), dtype=udt, device="cuda") for _ in range(2)]
        # first call on this state: no commit, pseudo-values into u[0]
        g.commit_verify(d["S"], d["path"], torch.zeros_like(d["plen"]), own, d["q"], d["k"],
                        d["v"], d["alpha"], d["beta"], d["parent"], out=d["out"],
                        u_out=d["u"][0], stream=stream)
        fused_u.append([g.commit_verify(d["S"], d["path"], d["plen"], own, d["q"], d["k"],
                                        d["v"], d["alpha"], d["beta"], d["parent"],
                                        out=d["out"], u_prev=d["u"][par],
                                        u_out=d["u"][1 - par], stream=stream, prepare=True)
                        for par in range(2)])
        seed_u16.append(g.commit_verify(d["S"], d["path"], torch.zeros_like(d["plen"]), own,
                                        d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                        d["parent"], out=d["out"], u_out=d["u16"][0],
                                        stream=stream, prepare=True))
        fused_u16.append([g.commit_verify(d["S"], d["path"], d["plen"], own, d["q"], d["k"],
                                          d["v"], d["alpha"], d["beta"], d["parent"],
                                          out=d["out"], u_prev=d["u16"][par],
                                          u_out=d["u16"][1 - par], stream=stream, prepare=True)
                          for par in range(2)])
        p = sets[(i - 1) % R]
        fused_solve.append(g.commit_verify(d["S"], p["path"], p["plen"],
                                           (p["k"], p["v"], p["alpha"], p["beta"], p["parent"]),
                                           d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                           d["parent"], out=d["out"], stream=stream,
                                           prepare=True))
        ver.append(g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"],
                            out=d["out"], stream=stream, prepare=True))
        com.append(g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"], d["alpha"], d["beta"],
                            d["parent"], stream=stream, prepare=True))
    visits = [0] * R

    def fused_step(i):
        fused_u[i][visits[i] & 1]()
        visits[i] += 1

    for i in range(args.warmup):
        fused_step(i % R)
    torch.cuda.synchronize()
    # Clocks settle only after some milliseconds of sustained load: without
    # this the first timed region runs ~10% slow whatever it holds.  Keep
    # stepping (untimed) until 30 ms of GPU time have passed.
    settle0, settle1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle0.record(stream)
    settled = 0
    while True:
        for i in range(100):
            fused_step(i % R)
        settle1.record(stream)
        settle1.synchronize()
        settled += 100
        if settle0.elapsed_time(settle1) >= 30.0 or settled >= 20000:
            break

    K = args.steps
    host_s = {}

    def timed(name, body):
        for i in range(2 * R):   # settle this launch shape before its timed region
            body(i % R)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        h0 = time.perf_counter()
        for i in range(K):
            body(i % R)
        host_s[name] = (time.perf_counter() - h0) / K
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    def separate(i):
        ver[i]()
        com[i]()

    visits16 = [0] * R

    def fused_step_u16(i):
        fused_u16[i][visits16[i] & 1]()
        visits16[i] += 1

    ms_step = timed("fused", fused_step)
    # the fp16 pseudo-value chain starts from a first call on each set's
    # current state
    for i in range(R):
        seed_u16[i]()
    u16_ms = timed("fused_u16", fused_step_u16)
    # back on the fp32 chain: reseed it from the current states
    for i, d in enumerate(sets):
        g.commit_verify(d["S"], d["path"], torch.zeros_like(d["plen"]),
                        (d["k"], d["v"], d["alpha"], d["beta"], d["parent"]), d["q"], d["k"],
                        d["v"], d["alpha"], d["beta"], d["parent"], out=d["out"],
                        u_out=d["u"][visits[i] & 1], stream=stream)
    solve_ms = timed("fused_solve", lambda i: fused_solve[i]())
    sep_ms = timed("separate", separate)
    ver_ms = timed("verify", lambda i: ver[i]())
    com_ms = timed("commit", lambda i: com[i]())
    recheck_ms = timed("fused_recheck", fused_step)
    log(f"fused {ms_step * 1e3:.2f} us (again at the end: {recheck_ms * 1e3:.2f} us; fp16 "
        f"pseudo-values: {u16_ms * 1e3:.2f} us; commit "
        f"solving for its pseudo-values: {solve_ms * 1e3:.2f} us), "
        f"separate {sep_ms * 1e3:.2f} us, verify {ver_ms * 1e3:.2f} "
        f"us, commit {com_ms * 1e3:.2f} us per launch (host enqueue "
        f"{host_s['fused'] * 1e6:.1f} us per fused launch)")
    nodes = batch * n
    mean_plen = float(np.mean([float(np.sum(d["plen_host"])) for d in sets]))
    vbytes = verify_bytes(batch, n, H, dk, dv)
    cbytes = commit_bytes(batch, H, dk, dv, [mean_plen])
    fbytes = fused_bytes(batch, n, H, dk, dv, [mean_plen])
    step_s = ms_step * 1e-3
    achieved = fbytes / step_s / 1e9
    traffic = read_traffic()

    # the acceptance walk and path extraction that produce the next step's
    # commit input (integer kernels, launch-latency bound), same trees
    ts0 = host0[0]
    draft, vtok = gs.make_accept_tokens(np.random.default_rng(0), ts0.parent, p_match=0.8)
    dpar, ddraft, dvtok = dev(ts0.parent), dev(draft), dev(vtok)
    acc_call = g.accept(dpar, ddraft, dvtok, stream=stream, prepare=True)
    acc_t, _, _ = acc_call()
    path_call = g.path(dpar, acc_t, max_path, stream=stream, prepare=True)

    def timed_call(call, reps=200):
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    accept_us = timed_call(acc_call)
    path_us = timed_call(path_call)
    # the step before verify: width-8 best-first construction of the same
    # batch's 64-node trees from a synthetic candidate table (K = 8)
    clp, ctok, croot = gs.candidate_table(np.random.default_rng(1), batch, n, 8)
    build_call = g.build_tree(dev(clp), dev(ctok), dev(croot), 8, 12, stream=stream,
                              prepare=True)
    build_us = timed_call(build_call)

    # tree-size-126 comparison: the tree verify against single-branch
    # recurrent verification (one chain per root-to-leaf branch) on the same
    # inputs, 8 rotating sets of width-8 best-first trees of 126 nodes
    cmp126 = b64 = None
    if not args.no_compare:
        sets = fused_u = fused_u16 = seed_u16 = fused_solve = ver = com = None
        torch.cuda.empty_cache()
        c_sets = []
        for s_ in range(8):
            ts = gs.make_tree126(s_)
            c_sets.append(dict(q=dev(ts.q_bits.view(np.int16)).view(torch.bfloat16),
                               k=dev(ts.k_bits.view(np.int16)).view(torch.bfloat16),
                               v=dev(ts.v_bits.view(np.int16)).view(torch.bfloat16),
                               alpha=dev(ts.alpha), beta=dev(ts.beta), parent=dev(ts.parent),
                               S=dev(ts.S0), leaves=sum(len(gs.leaves(p)) for p in ts.parent),
                               steps=sum(branch_node_steps(p) for p in ts.parent)))
        for d in c_sets:
            d["out"] = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
        tv126 = [g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"],
                          out=d["out"], stream=stream, prepare=True) for d in c_sets]
        bv126 = [g.branch_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                                 d["S"], out=d["out"], stream=stream, prepare=True)
                 for d in c_sets]

        def timed_list(calls, reps):
            for i in range(3):
                calls[i % len(calls)]()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                calls[i % len(calls)]()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        t_tree = timed_list(tv126, 40)
        t_branch = timed_list(bv126, 10)
        w126 = gs.TREE126
        # what the branch baseline computes: per branch node and head,
        # w = S^T k (2 d^2 flops), the update alpha S + (beta k)(v - alpha w)^T
        # (3 d^2) and o = S^T q (2 d^2); on the fp32 vector peak this is a
        # floor for any recurrent branch verify on this chip
        steps = float(np.mean([d["steps"] for d in c_sets]))   # per set, all sequences
        branch_flop = steps * w126.H * 7 * w126.d_k * w126.d_v
        floor_us = branch_flop / FP32_VECTOR_PEAK * 1e6
        cmp126 = {"workload": w126.name, "tree_verify_us": t_tree, "branch_verify_us": t_branch,
                  "speedup": t_branch / t_tree,
                  "branch_node_steps_per_tree": steps / w126.batch,
                  "branch_tflop_per_s": branch_flop / (t_branch * 1e-6) / 1e12,
                  "branch_fp32_floor_us": floor_us,
                  "speedup_vs_branch_floor": floor_us / t_tree,
                  "mean_leaves_per_tree": float(np.mean([d["leaves"] / w126.batch
                                                         for d in c_sets])),
                  "tree_verify_nodes_per_s": w126.batch * w126.n / (t_tree * 1e-6),
                  "pages_speedup_b200": 7.1}
        log(f"n=126: tree verify {t_tree:.1f} us, branch verify {t_branch:.1f} us, "
            f"speedup {t_branch / t_tree:.2f} (branch at {cmp126['branch_tflop_per_s']:.1f} "
            f"TFLOP/s; its fp32 floor {floor_us:.0f} us, {floor_us / t_tree:.2f}x the tree)")
        c_sets = tv126 = bv126 = None

        # the batch-64, 128-node workload (a quarter chains, a quarter stars
        # and 16-ary bushes, half random recursive trees): verify and the
        # commit of each sequence's accepted branch, 2 rotating sets of
        # ~0.6 GB each
        torch.cuda.empty_cache()
        w3 = gs.WORKLOADS[3]
        b_sets = []
        for s_ in range(2):
            ts = gs.make_config(3, s=s_)
            pth, pl = ts.paths(max_path=w3.n)
            b_sets.append(dict(q=dev(ts.q_bits.view(np.int16)).view(torch.bfloat16),
                               k=dev(ts.k_bits.view(np.int16)).view(torch.bfloat16),
                               v=dev(ts.v_bits.view(np.int16)).view(torch.bfloat16),
                               alpha=dev(ts.alpha), beta=dev(ts.beta), parent=dev(ts.parent),
                               S=dev(ts.S0), path=dev(pth), plen=dev(pl),
                               m=float(np.sum(pl))))
            b_sets[-1]["out"] = torch.empty((w3.batch, w3.n, w3.H, w3.d_v), dtype=torch.float32,
                                            device="cuda")
        vb = [g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S"],
                       out=d["out"], stream=stream, prepare=True) for d in b_sets]
        cb = [g.commit(d["S"], d["path"], d["plen"], d["k"], d["v"], d["alpha"], d["beta"],
                       d["parent"], stream=stream, prepare=True) for d in b_sets]
        t_vb = timed_list(vb, 20)
        t_cb = timed_list(cb, 20)
        vb_bytes = verify_bytes(w3.batch, w3.n, w3.H, w3.d_k, w3.d_v)
        cb_bytes = commit_bytes(w3.batch, w3.H, w3.d_k, w3.d_v,
                                [float(np.mean([d["m"] for d in b_sets]))])
        b64 = {"workload": w3.name, "verify_us": t_vb, "commit_us": t_cb,
               "verify_nodes_per_s": w3.batch * w3.n / (t_vb * 1e-6),
               "verify_hbm_gbps": vb_bytes / (t_vb * 1e-6) / 1e9,
               "commit_hbm_gbps": cb_bytes / (t_cb * 1e-6) / 1e9,
               "verify_algorithmic_bytes": vb_bytes, "commit_algorithmic_bytes": cb_bytes}
        log(f"b64/n128: verify {t_vb:.1f} us ({b64['verify_hbm_gbps']:.0f} GB/s), commit "
            f"{t_cb:.1f} us ({b64['commit_hbm_gbps']:.0f} GB/s)")
        b_sets = vb = cb = None

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
                   "step": "commit the accepted path (pseudo-values carried from the previous "
                           "verify) + verify the trees, writing their pseudo-values (one launch)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "gdn_tree_commit_verify", "algorithmic_bytes_per_launch": fbytes,
                     "mean_launch_us": step_s * 1e6},
        "fused_u16_us": u16_ms * 1e3,
        "fused_commit_solving_us": solve_ms * 1e3,
        "separate_step_us": sep_ms * 1e3,
        "separate_step_nodes_per_s": nodes / (sep_ms * 1e-3),
        "verify_us": ver_ms * 1e3,
        "commit_us": com_ms * 1e3,
        "verify_nodes_per_s": nodes / (ver_ms * 1e-3),
        "verify_hbm_gbps": vbytes / (ver_ms * 1e-3) / 1e9,
        "commit_hbm_gbps": cbytes / (com_ms * 1e-3) / 1e9,
        "host_enqueue_us_per_step": host_s["fused"] * 1e6,
        "copy_gbps": copy_gbps,
        "tree_build_us": build_us,
        "accept_us": accept_us,
        "path_us": path_us,
        "tree126_vs_branch": cmp126,
        "b64_n128": b64,
    }
    if not args.no_cpu_baseline:
        ts, path, plen = host0
        result["cpu_baseline"] = cpu_baseline(ts, path, plen)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
