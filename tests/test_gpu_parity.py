"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Gates (max|gpu - ref| / max|ref| over a whole output tensor):
  2e-3 for bf16 q/k/v with fp32 state and accumulation, 1e-5 all-fp32;
  integer outputs (status, depth, ancestor masks, paths) bit-exact.
"""
import numpy as np
import pytest
import torch

import gdn_synth as gs
import oracle
from gpu_util import dev, host, upload

pytestmark = pytest.mark.gpu

BF16_GATE = 2e-3
FP32_GATE = 1e-5


def gate(ts):
    return BF16_GATE if ts.dtype == "bf16" else FP32_GATE


def say(*a):
    print(*a, flush=True)


def run_verify(g, ts, status=True):
    d = upload(ts)
    st = torch.full((ts.parent.shape[0],), -7, dtype=torch.int32, device="cuda") if status else None
    out = g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"], status=st)
    torch.cuda.synchronize()
    return host(out), (host(st) if status else None), d


# ---------------------------------------------------------------------------
# verify parity on the five workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("chain", [False, True])
def test_verify_tiny_fp32(gpu_lib, chain):
    say("verify tiny fp32 chain=", chain)
    ts = gs.make_config(0, chain=chain)
    out, st, _ = run_verify(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0]
    assert oracle.rel_err(out, ref) <= FP32_GATE


def test_verify_layer_b1_n32(gpu_lib):
    say("verify b1 n32 bf16")
    ts = gs.make_config(1)
    out, st, _ = run_verify(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist()
    err = oracle.rel_err(out, ref)
    say("rel err", err)
    assert err <= BF16_GATE


def test_verify_layer_b16_n64_full(gpu_lib):
    """the benchmarked workload, whole output tensor"""
    say("verify b16 n64 bf16 full")
    ts = gs.make_config(2)
    out, st, _ = run_verify(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0] * 16
    err = oracle.rel_err(out, ref)
    say("rel err", err)
    assert err <= BF16_GATE


@pytest.mark.parametrize("layer", [0, 47])
def test_stack_layer_verify_commit(gpu_lib, layer):
    """one layer of the 48-layer stack through the separate verify and commit
    kernels, whole tensors (the stacked fused run is in test_gpu_deep.py)"""
    say("stack layer", layer)
    ts = gs.make_config(4, layer=layer)
    out, st, d = run_verify(gpu_lib, ts)
    path, plen = ts.paths(max_path=13)
    S = d["S0"].clone()
    cst = torch.full((32,), -7, dtype=torch.int32, device="cuda")
    gpu_lib.commit(S, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                   status=cst)
    torch.cuda.synchronize()
    ref, _ = oracle.verify_set(ts)
    assert oracle.rel_err(out, ref) <= BF16_GATE
    Sref, rst = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert host(cst).tolist() == rst.tolist() == [0] * 32
    assert oracle.rel_err(host(S), Sref) <= BF16_GATE


# ---------------------------------------------------------------------------
# shapes: ragged n, every supported head dim, n = 1, forests
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,dk,dv,dtype,H,batch", [
    (1, 16, 16, "fp32", 2, 3),
    (1, 128, 128, "bf16", 4, 2),
    (37, 32, 64, "fp32", 3, 2),
    (37, 128, 128, "bf16", 5, 3),
    (64, 128, 128, "bf16", 3, 2),
    (100, 64, 48, "bf16", 2, 2),
    (128, 128, 128, "bf16", 2, 2),
    (128, 8, 128, "fp32", 1, 1),
    (65, 128, 128, "bf16", 2, 2),
    (17, 24, 40, "fp32", 2, 2),
])
def test_verify_shapes(gpu_lib, n, dk, dv, dtype, H, batch):
    say("shape", n, dk, dv, dtype, H, batch)
    rng = np.random.default_rng(n * 1000 + dk + dv)
    par = np.stack([gs.random_recursive_tree(rng, n, max_depth=int(rng.integers(1, 20)))
                    for _ in range(batch)])
    if batch > 1 and n > 4:
        par[1, n // 2] = -1                   # forest: a second root
    ts = gs.make_set(par, H, dk, dv, dtype, seed=n + dk)
    out, st, _ = run_verify(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0] * batch
    assert oracle.rel_err(out, ref) <= gate(ts)


@pytest.mark.parametrize("shape", ["chain", "star", "bfs16"])
def test_verify_extreme_trees_n128(gpu_lib, shape):
    say("extreme", shape)
    par = {"chain": gs.chain_tree(128), "star": gs.star_tree(128),
           "bfs16": gs.kary_bfs_tree(128, 16)}[shape]
    ts = gs.make_set(np.stack([par, par]), 4, 128, 128, "bf16", seed=5)
    out, _, _ = run_verify(gpu_lib, ts)
    ref, _ = oracle.verify_set(ts)
    assert oracle.rel_err(out, ref) <= BF16_GATE


def test_verify_fp32_gate_at_d128(gpu_lib):
    """all-fp32 inputs at the full head size meet the fp32 gate"""
    ts = gs.make_set(gs.make_trees(1, np.random.default_rng(3)), 4, 128, 128, "fp32", seed=3)
    out, _, _ = run_verify(gpu_lib, ts)
    ref, _ = oracle.verify_set(ts)
    assert oracle.rel_err(out, ref) <= FP32_GATE


# ---------------------------------------------------------------------------
# commit parity, commit-then-verify, invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,max_path", [(0, None), (1, None), (2, None), (1, 9), (2, 13)])
def test_commit_parity(gpu_lib, cfg, max_path):
    """max_path None: the tree size (32-slot chunks); 9 and 13 (the deepest
    path of those trees): the one-chunk kernel for paths of at most 16 nodes"""
    say("commit cfg", cfg, "max_path", max_path)
    ts = gs.make_config(cfg)
    d = upload(ts)
    path, plen = ts.paths(max_path=ts.parent.shape[1] if max_path is None else max_path)
    S = d["S0"].clone()
    st = torch.full((ts.parent.shape[0],), -7, dtype=torch.int32, device="cuda")
    gpu_lib.commit(S, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                   status=st)
    torch.cuda.synchronize()
    Sref, rst = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert host(st).tolist() == rst.tolist()
    assert oracle.rel_err(host(S), Sref) <= gate(ts)


def test_commit_deep_chain_n128(gpu_lib):
    ts = gs.make_set(np.stack([gs.chain_tree(128)] * 2), 2, 128, 128, "bf16", seed=8,
                     accepted=np.array([127, 64], np.int32))
    d = upload(ts)
    path, plen = ts.paths(max_path=128)
    S = d["S0"].clone()
    gpu_lib.commit(S, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"])
    Sref, _ = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert oracle.rel_err(host(S), Sref) <= BF16_GATE


def test_commit_chunk_edges_n128(gpu_lib):
    """the 32-slot chunked commit at path lengths on and next to the chunk
    edges (1, 32, 33, 64, 96, 97 nodes), the next chunk's rows prefetched"""
    ts = gs.make_set(np.stack([gs.chain_tree(128)] * 6), 2, 128, 128, "bf16", seed=12,
                     accepted=np.array([0, 31, 32, 63, 95, 96], np.int32))
    d = upload(ts)
    path, plen = ts.paths(max_path=128)
    assert plen.tolist() == [1, 32, 33, 64, 96, 97]
    S = d["S0"].clone()
    st = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    gpu_lib.commit(S, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                   status=st)
    torch.cuda.synchronize()
    Sref, rst = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert host(st).tolist() == rst.tolist() == [0] * 6
    assert oracle.rel_err(host(S), Sref) <= BF16_GATE


def test_commit_then_verify_subtree(gpu_lib):
    """the committed state, verified over the re-rooted subtree below the
    accepted node, reproduces the original verify outputs of that subtree"""
    ts = gs.make_config(1)
    par = ts.parent[0]
    a = next(i for i in range(1, len(par)) if (par == i).sum() >= 2)
    out, _, d = run_verify(gpu_lib, ts)
    p = gs.path_to(par, a)[None].astype(np.int32)
    S = d["S0"].clone()
    gpu_lib.commit(S, dev(p), dev(np.array([p.shape[1]], np.int32)), d["k"], d["v"], d["alpha"],
                   d["beta"], d["parent"])
    desc = [i for i in range(len(par)) if i != a and a in set(gs.path_to(par, i))]
    m = {o: j for j, o in enumerate(desc)}
    newp = np.array([-1 if par[o] == a else m[par[o]] for o in desc], np.int32)[None]
    sl = lambda x: x[:, desc].contiguous()
    o2 = gpu_lib.verify(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["alpha"]), sl(d["beta"]),
                        dev(newp), S)
    torch.cuda.synchronize()
    assert oracle.rel_err(host(o2), out[:, desc]) <= BF16_GATE


def test_verify_leaves_state_untouched_and_is_deterministic(gpu_lib):
    ts = gs.make_config(2)
    d = upload(ts)
    before = d["S0"].clone()
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"])
    o1 = gpu_lib.verify(*args)
    o2 = gpu_lib.verify(*args)
    torch.cuda.synchronize()
    assert torch.equal(d["S0"], before)
    assert torch.equal(o1, o2)


def _verify_with(g, d, **over):
    x = dict(d)
    x.update(over)
    out = g.verify(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["parent"], x["S0"])
    torch.cuda.synchronize()
    return host(out)


def test_homogeneity_bitwise_on_gpu(gpu_lib):
    """the outputs are linear in (V, S0) jointly; doubling both is exact in
    floating point (and in the hi / lo splits), so the outputs double bit
    for bit (MFMA kernel, bf16)"""
    ts = gs.make_config(2, batch=4, heads=8)
    d = upload(ts)
    o1 = _verify_with(gpu_lib, d)
    o2 = _verify_with(gpu_lib, d, v=(d["v"].float() * 2).to(torch.bfloat16), S0=d["S0"] * 2)
    assert np.array_equal(o2, 2 * o1)


def test_additivity_on_gpu(gpu_lib):
    """out(V1 + V2, S1 + S2) = out(V1, S1) + out(V2, S2) for one tree (fp32
    path: the sums are formed in fp32, so to within their rounding)"""
    A = gs.make_config(1, heads=8)
    a, b = gs.make_set(A.parent, 8, 128, 128, "fp32", seed=3), gs.make_set(A.parent, 8, 128, 128,
                                                                           "fp32", seed=4)
    da, db = upload(a), upload(b)
    o_a = _verify_with(gpu_lib, da)
    o_b = _verify_with(gpu_lib, da, v=db["v"], S0=db["S0"])
    o_ab = _verify_with(gpu_lib, da, v=da["v"] + db["v"], S0=da["S0"] + db["S0"])
    assert oracle.rel_err(o_ab, o_a + o_b) <= 1e-5


def test_non_descendants_unchanged_on_gpu(gpu_lib):
    """new inputs at one node change the outputs of that node's subtree only;
    every other node's output is bit-identical (its X and Y entries for the
    node are masked to exact zeros)"""
    ts = gs.make_config(2, batch=4, heads=8)
    d = upload(ts)
    o1 = _verify_with(gpu_lib, d)
    j = 10
    rng = np.random.default_rng(5)
    d2 = {key: t.clone() for key, t in d.items()}
    for key in ("q", "k", "v"):
        x = torch.from_numpy(rng.standard_normal(d2[key][:, j].shape).astype(np.float32))
        if key != "v":
            x = x / x.norm(dim=-1, keepdim=True)
        d2[key][:, j] = x.to(d2[key].dtype).cuda()
    d2["alpha"][:, j] = 0.5
    d2["beta"][:, j] = 0.9
    o2 = _verify_with(gpu_lib, d2)
    for b in range(ts.parent.shape[0]):
        par = ts.parent[b]
        sub = np.zeros(len(par), bool)
        sub[j] = True
        for i in range(j + 1, len(par)):
            sub[i] = par[i] >= 0 and sub[par[i]]
        assert np.array_equal(o1[b, ~sub], o2[b, ~sub]), b
        assert not np.array_equal(o1[b, sub], o2[b, sub]), b


def test_closed_forms_on_gpu(gpu_lib):
    """beta = 0: o_i = e^{g_i} S0^T q_i (a plain product times the path decay;
    MFMA kernel, bf16); q = k, beta = 1 with unit keys: o = v for any alpha
    and S0 (fp32 path)"""
    ts = gs.make_config(2, batch=4, heads=8)
    d = upload(ts)
    o = _verify_with(gpu_lib, d, beta=torch.zeros_like(d["beta"]))
    la = np.log(ts.alpha.astype(np.float64))
    ref = np.empty(o.shape)
    for b in range(ts.parent.shape[0]):
        g = np.zeros((ts.parent.shape[1], ts.alpha.shape[2]))
        for i, p in enumerate(ts.parent[b]):
            g[i] = la[b, i] + (g[p] if p >= 0 else 0.0)
        qs = np.einsum("nhk,hkv->nhv", ts.q[b].astype(np.float64), ts.S0[b].astype(np.float64))
        ref[b] = np.exp(g)[:, :, None] * qs
    assert oracle.rel_err(o, ref) <= 2e-5
    f = gs.make_set(ts.parent, 8, 128, 128, "fp32", seed=6)
    df = upload(f)
    o = _verify_with(gpu_lib, df, q=df["k"], beta=torch.ones_like(df["beta"]))
    assert oracle.rel_err(o, f.v) <= 1e-5


def test_relabeling_on_gpu(gpu_lib):
    ts = gs.make_config(1)
    out, _, d = run_verify(gpu_lib, ts)
    rng = np.random.default_rng(2)
    par = ts.parent[0]
    n = len(par)
    order, ready = [], [0]
    while ready:
        j = ready.pop(int(rng.integers(0, len(ready))))
        order.append(j)
        ready += [c for c in range(n) if par[c] == j]
    perm = np.array(order)
    inv = np.empty(n, int)
    inv[perm] = np.arange(n)
    newp = np.array([-1 if par[o] < 0 else inv[par[o]] for o in perm], np.int32)[None]
    sl = lambda x: x[:, perm].contiguous()
    o2 = gpu_lib.verify(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["alpha"]), sl(d["beta"]),
                        dev(newp), d["S0"])
    assert oracle.rel_err(host(o2), out[:, perm]) <= BF16_GATE


# ---------------------------------------------------------------------------
# faults
# ---------------------------------------------------------------------------
def test_verify_bad_parent(gpu_lib):
    ts = gs.make_config(2, batch=3)
    ts.parent[1, 10] = 12
    ts.parent[2, 0] = -2
    out, st, _ = run_verify(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0, 1, 1]
    assert np.isnan(out[1:]).all() and np.isfinite(out[0]).all()
    assert oracle.rel_err(out[0], ref[0]) <= BF16_GATE


@pytest.mark.parametrize("n", [65, 128])
def test_verify_bad_parent_n128(gpu_lib, n):
    """the 65..128-node kernel: a node that is its own parent, a parent
    after its node; the healthy sequence is unaffected"""
    say("verify bad parent n", n)
    rng = np.random.default_rng(n + 77)
    par = np.stack([gs.random_recursive_tree(rng, n, max_depth=16) for _ in range(3)])
    par[1, n - 1] = n - 1
    par[2, 40] = n - 1
    ts = gs.make_set(par, 4, 128, 128, "bf16", seed=n)
    out, st, _ = run_verify(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0, 1, 1]
    assert np.isnan(out[1:]).all() and np.isfinite(out[0]).all()
    assert oracle.rel_err(out[0], ref[0]) <= BF16_GATE


def test_commit_bad_paths_leave_state(gpu_lib):
    ts = gs.make_config(2, batch=4)
    d = upload(ts)
    path, plen = ts.paths(max_path=16)
    path[0, 1] = 64                     # id out of range
    path[1, 0] = path[1, 1]             # not starting at a root
    plen[2] = 17                        # longer than max_path
    S = d["S0"].clone()
    st = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    gpu_lib.commit(S, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                   status=st)
    torch.cuda.synchronize()
    Sref, rst = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert host(st).tolist() == rst.tolist() == [2, 2, 2, 0]
    assert torch.equal(S[:3], d["S0"][:3])
    assert oracle.rel_err(host(S)[3], Sref[3]) <= BF16_GATE


def test_commit_empty_path_is_noop(gpu_lib):
    ts = gs.make_config(1)
    d = upload(ts)
    S = d["S0"].clone()
    gpu_lib.commit(S, dev(np.full((1, 4), -1, np.int32)), dev(np.zeros(1, np.int32)), d["k"],
                   d["v"], d["alpha"], d["beta"], d["parent"])
    torch.cuda.synchronize()
    assert torch.equal(S, d["S0"])


# ---------------------------------------------------------------------------
# single-branch recurrent baseline: the same outputs as the tree verify
# ---------------------------------------------------------------------------
def run_branch(g, ts):
    d = upload(ts)
    st = torch.full((ts.parent.shape[0],), -7, dtype=torch.int32, device="cuda")
    out = g.branch_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"],
                          status=st)
    torch.cuda.synchronize()
    return host(out), host(st), d


@pytest.mark.parametrize("cfg,chain", [(0, False), (0, True), (1, False), (2, False)])
def test_branch_verify_parity(gpu_lib, cfg, chain):
    say("branch verify cfg", cfg, "chain", chain)
    ts = gs.make_config(cfg, chain=chain)
    out, st, _ = run_branch(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist()
    err = oracle.rel_err(out, ref)
    say("rel err", err)
    assert err <= gate(ts)


def test_branch_verify_tree126_sampled(gpu_lib):
    """the comparison workload (126-node width-8 best-first trees), full
    launch, checked on four sequences"""
    ts = gs.make_tree126(0)
    out, st, _ = run_branch(gpu_lib, ts)
    assert st.tolist() == [0] * 16
    pick = [0, 5, 10, 15]
    ref, _ = oracle.verify_set(gs.select(ts, pick))
    assert oracle.rel_err(out[pick], ref) <= BF16_GATE


@pytest.mark.parametrize("shape", ["chain", "star", "bfs16"])
def test_branch_verify_extreme_trees(gpu_lib, shape):
    par = {"chain": gs.chain_tree(128), "star": gs.star_tree(128),
           "bfs16": gs.kary_bfs_tree(128, 16)}[shape]
    ts = gs.make_set(np.stack([par, par]), 2, 128, 128, "bf16", seed=11)
    out, _, _ = run_branch(gpu_lib, ts)
    ref, _ = oracle.verify_set(ts)
    assert oracle.rel_err(out, ref) <= BF16_GATE


def test_branch_verify_shapes_and_faults(gpu_lib):
    rng = np.random.default_rng(12)
    par = np.stack([gs.random_recursive_tree(rng, 37, max_depth=9) for _ in range(3)])
    par[1, 20] = 25
    ts = gs.make_set(par, 3, 48, 40, "fp32", seed=12)
    out, st, _ = run_branch(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0, 1, 0]
    assert np.isnan(out[1]).all()
    for b in (0, 2):
        assert oracle.rel_err(out[b], ref[b]) <= FP32_GATE


# ---------------------------------------------------------------------------
# fused commit (previous tree's path) + verify (next tree)
# ---------------------------------------------------------------------------
def run_commit_verify(g, prev, cur, path, plen):
    dp, dc = upload(prev), upload(cur)
    S = dp["S0"].clone()
    st = torch.full((cur.parent.shape[0],), -7, dtype=torch.int32, device="cuda")
    out = g.commit_verify(S, dev(path), dev(plen),
                          (dp["k"], dp["v"], dp["alpha"], dp["beta"], dp["parent"]),
                          dc["q"], dc["k"], dc["v"], dc["alpha"], dc["beta"], dc["parent"],
                          status=st)
    torch.cuda.synchronize()
    return host(out), host(S), host(st)


def oracle_commit_verify(prev, cur, path, plen):
    """the definition: commit along the previous tree's path, then verify the
    next tree from the committed state"""
    Sref, cst = oracle.commit_set(prev, path_arr=path, path_len=plen)
    oref, vst = oracle.verify(cur.q, cur.k, cur.v, cur.alpha, cur.beta, cur.parent, Sref)
    return oref, Sref, cst | vst


def test_commit_verify_b16_n64_full(gpu_lib):
    """the benchmarked step: two consecutive trees of the b16/n64 workload"""
    say("commit-verify b16 n64")
    prev, cur = gs.make_config(2, s=0), gs.make_config(2, s=1)
    path, plen = prev.paths(max_path=13)
    out, S, st = run_commit_verify(gpu_lib, prev, cur, path, plen)
    oref, Sref, rst = oracle_commit_verify(prev, cur, path, plen)
    assert st.tolist() == rst.tolist() == [0] * 16
    eo, es = oracle.rel_err(out, oref), oracle.rel_err(S, Sref)
    say("rel err out", eo, "S", es)
    assert eo <= BF16_GATE and es <= BF16_GATE


def test_commit_verify_matches_separate_calls(gpu_lib):
    """same tensors for both trees; the fused call agrees with commit then
    verify (the same stages, so to within rounding order) and with the oracle"""
    ts = gs.make_config(1)
    d = upload(ts)
    path, plen = ts.paths(max_path=32)
    out, S, st = run_commit_verify(gpu_lib, ts, ts, path, plen)
    S2 = d["S0"].clone()
    gpu_lib.commit(S2, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"])
    o2 = gpu_lib.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], S2)
    torch.cuda.synchronize()
    assert st.tolist() == [0]
    say("fused == separate:", np.array_equal(S, host(S2)), np.array_equal(out, host(o2)))
    assert oracle.rel_err(S, host(S2)) <= 1e-6
    assert oracle.rel_err(out, host(o2)) <= 1e-5
    oref, Sref, _ = oracle_commit_verify(ts, ts, path, plen)
    assert oracle.rel_err(out, oref) <= BF16_GATE


@pytest.mark.parametrize("n_prev,n,dk,dv,dtype,max_path", [
    (128, 64, 128, 128, "bf16", None),   # fused kernel, four commit chunks
    (20, 1, 128, 128, "bf16", None),     # fused kernel, one-node tree
    (64, 64, 128, 128, "bf16", 13),      # fused kernel, paths within the first chunk
    (64, 100, 128, 128, "bf16", None),   # 65..128-node fused kernel, 32-slot chunks
    (8, 65, 128, 128, "bf16", None),     # 65..128-node fused kernel, one 16-slot chunk
    (37, 37, 64, 64, "fp32", None),      # generic commit + generic verify
    (40, 64, 128, 128, "fp32", None),    # fp32-MFMA commit, then fp32-MFMA verify ORing its flag
    (50, 30, 32, 48, "bf16", None),
])
def test_commit_verify_shapes_and_faults(gpu_lib, n_prev, n, dk, dv, dtype, max_path):
    """sequence 0 clean, 1 bad previous path, 2 bad new tree, 3 both, 4 empty path"""
    say("commit-verify", n_prev, n, dk, dv, dtype, max_path)
    rng = np.random.default_rng(n_prev * 7 + n)
    pp = np.stack([gs.chain_tree(n_prev) if n_prev == 128 else
                   gs.random_recursive_tree(rng, n_prev, max_depth=12) for _ in range(5)])
    pc = np.stack([gs.random_recursive_tree(rng, n, max_depth=10) for _ in range(5)])
    acc = np.array([gs.pick_leaf(rng, pp[i]) for i in range(5)], np.int32)
    if n_prev == 128:
        acc[:] = 127
    prev = gs.make_set(pp, 2, dk, dv, dtype, seed=n_prev, accepted=acc)
    cur = gs.make_set(pc, 2, dk, dv, dtype, seed=n_prev + 1)
    path, plen = prev.paths(max_path=n_prev if max_path is None else max_path)
    path[1, plen[1] - 1] = n_prev       # id out of range
    path[3, 0] = n_prev + 3
    plen[4] = 0
    cur.parent[2, n - 1] = n - 1        # parent not before the node
    cur.parent[3, 0] = -5
    out, S, st = run_commit_verify(gpu_lib, prev, cur, path, plen)
    oref, Sref, rst = oracle_commit_verify(prev, cur, path, plen)
    assert st.tolist() == rst.tolist() == [0, 2, 1, 3, 0]
    for b in (1, 3, 4):
        assert np.array_equal(S[b], prev.S0[b]), b
    assert np.isnan(out[2:4]).all()
    g = gate(prev)
    for b in (0, 2):
        assert oracle.rel_err(S[b], Sref[b]) <= g, b
    for b in (0, 1, 4):
        assert oracle.rel_err(out[b], oref[b]) <= g, b


# ---------------------------------------------------------------------------
# fused step with pseudo-values carried from one call to the next
# ---------------------------------------------------------------------------
U_DTYPES = {"fp32": torch.float32, "fp16": torch.float16}


@pytest.mark.parametrize("udt", ["fp32", "fp16"])
def test_commit_verify_pseudo_values_decode_loop(gpu_lib, udt):
    """call 1 verifies tree A (no commit) and writes its u; call 2 commits
    A's accepted path from that u (no solve) and verifies tree B; every
    output against the oracle.  fp16 pseudo-values are the fp32 ones
    rounded to nearest, bit for bit."""
    say("commit-verify with pseudo-values", udt)
    A, B = gs.make_config(2, s=5), gs.make_config(2, s=6)
    dA, dB = upload(A), upload(B)
    S = dA["S0"].clone()
    prevA = (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"])
    uA = torch.full(dA["v"].shape, 7.0, dtype=U_DTYPES[udt], device="cuda")
    uB = torch.full(dB["v"].shape, 7.0, dtype=U_DTYPES[udt], device="cuda")
    st = torch.full((16,), -7, dtype=torch.int32, device="cuda")
    zero = dev(np.zeros(16, np.int32))
    pathA, plenA = A.paths(max_path=13)
    outA = gpu_lib.commit_verify(S, dev(pathA), zero, prevA, dA["q"], dA["k"], dA["v"],
                                 dA["alpha"], dA["beta"], dA["parent"], u_out=uA, status=st)
    torch.cuda.synchronize()
    refA, _ = oracle.verify_set(A)
    UA, _ = oracle.pseudo_set(A)
    assert host(st).tolist() == [0] * 16 and torch.equal(S, dA["S0"])
    assert oracle.rel_err(host(outA), refA) <= BF16_GATE
    eu = oracle.rel_err(host(uA), UA)
    say("u rel err", eu)
    assert eu <= BF16_GATE
    if udt == "fp16":
        u32 = torch.empty(dA["v"].shape, dtype=torch.float32, device="cuda")
        S2 = dA["S0"].clone()
        gpu_lib.commit_verify(S2, dev(pathA), zero, prevA, dA["q"], dA["k"], dA["v"],
                              dA["alpha"], dA["beta"], dA["parent"], u_out=u32)
        torch.cuda.synchronize()
        assert torch.equal(uA.view(torch.int16), u32.half().view(torch.int16))
    outB = gpu_lib.commit_verify(S, dev(pathA), dev(plenA), prevA, dB["q"], dB["k"], dB["v"],
                                 dB["alpha"], dB["beta"], dB["parent"], u_prev=uA, u_out=uB,
                                 status=st)
    torch.cuda.synchronize()
    oref, Sref, rst = oracle_commit_verify(A, B, pathA, plenA)
    UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert host(st).tolist() == rst.tolist() == [0] * 16
    es, eo, eu = (oracle.rel_err(host(S), Sref), oracle.rel_err(host(outB), oref),
                  oracle.rel_err(host(uB), UB))
    say("rel err S", es, "out", eo, "u", eu)
    assert es <= BF16_GATE and eo <= BF16_GATE and eu <= BF16_GATE


@pytest.mark.parametrize("udt", ["fp32", "fp16"])
def test_commit_verify_decode_chain(gpu_lib, udt):
    """six decode steps on one state, 8 sequences x 8 heads of the b16/n64
    workload's trees: step t commits tree t-1's accepted path from the
    pseudo-values step t-1 wrote, then verifies tree t.  The committed state
    and every step's outputs track the oracle run along the same chain
    (commit then verify, fp64), within the gate at every step: the rounding
    of carried fp16 pseudo-values does not build up."""
    say("decode chain", udt)
    trees = [gs.make_config(2, s=20 + t, batch=8, heads=8) for t in range(6)]
    dev_sets = [upload(ts) for ts in trees]
    S = dev_sets[0]["S0"].clone()
    Sref = trees[0].S0.astype(np.float64)
    u = [torch.empty(dev_sets[0]["v"].shape, dtype=U_DTYPES[udt], device="cuda") for _ in range(2)]
    st = torch.full((8,), -7, dtype=torch.int32, device="cuda")
    worst_s = worst_o = 0.0
    for t, (ts, d) in enumerate(zip(trees, dev_sets)):
        prev_ts, prev_d = (trees[t - 1], dev_sets[t - 1]) if t else (ts, d)
        path, plen = prev_ts.paths(max_path=13)
        if t == 0:
            plen = np.zeros_like(plen)
        prev = (prev_d["k"], prev_d["v"], prev_d["alpha"], prev_d["beta"], prev_d["parent"])
        out = gpu_lib.commit_verify(S, dev(path), dev(plen), prev, d["q"], d["k"], d["v"],
                                    d["alpha"], d["beta"], d["parent"],
                                    u_prev=u[(t - 1) % 2] if t else None, u_out=u[t % 2],
                                    status=st)
        torch.cuda.synchronize()
        if t:
            Sref, cst = oracle.commit(Sref, path, plen, prev_ts.k, prev_ts.v, prev_ts.alpha,
                                      prev_ts.beta, prev_ts.parent)
            assert cst.tolist() == [0] * 8
        oref, vst = oracle.verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, Sref)
        assert host(st).tolist() == vst.tolist() == [0] * 8
        es, eo = oracle.rel_err(host(S), Sref), oracle.rel_err(host(out), oref)
        worst_s, worst_o = max(worst_s, es), max(worst_o, eo)
        assert es <= BF16_GATE and eo <= BF16_GATE, (t, es, eo)
    say("worst rel err over the chain: S", worst_s, "out", worst_o)


@pytest.mark.parametrize("udt", ["fp32", "fp16"])
def test_commit_verify_pseudo_values_long_path_and_faults(gpu_lib, udt):
    """a 64-node chain (two 32-slot chunks of known u), a bad path (state
    untouched) and a malformed new tree (NaN outputs and u)"""
    chain = gs.chain_tree(64)
    rng = np.random.default_rng(31)
    pcur = np.stack([gs.random_recursive_tree(rng, 40, max_depth=9) for _ in range(3)])
    A = gs.make_set(np.stack([chain] * 3), 2, 128, 128, "bf16", seed=31,
                    accepted=np.full(3, 63, np.int32))
    B = gs.make_set(pcur, 2, 128, 128, "bf16", seed=32)
    B.parent[2, 10] = 20
    dA, dB = upload(A), upload(B)
    S = dA["S0"].clone()
    prevA = (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"])
    uA = torch.empty(dA["v"].shape, dtype=U_DTYPES[udt], device="cuda")
    uB = torch.empty(dB["v"].shape, dtype=U_DTYPES[udt], device="cuda")
    path, plen = A.paths(max_path=64)
    gpu_lib.commit_verify(S, dev(path), dev(np.zeros(3, np.int32)), prevA, dA["q"], dA["k"],
                          dA["v"], dA["alpha"], dA["beta"], dA["parent"], u_out=uA)
    path[1, 5] = 70                                   # sequence 1: invalid path
    st = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    outB = gpu_lib.commit_verify(S, dev(path), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                                 dB["alpha"], dB["beta"], dB["parent"], u_prev=uA, u_out=uB,
                                 status=st)
    torch.cuda.synchronize()
    oref, Sref, rst = oracle_commit_verify(A, B, path, plen)
    assert host(st).tolist() == rst.tolist() == [0, 2, 1]
    Sh, oh, uh = host(S), host(outB), host(uB)
    assert np.array_equal(Sh[1], A.S0[1])
    assert oracle.rel_err(Sh[[0, 2]], Sref[[0, 2]]) <= BF16_GATE
    assert oracle.rel_err(oh[[0, 1]], oref[[0, 1]]) <= BF16_GATE
    assert np.isnan(oh[2]).all() and np.isnan(uh[2]).all()
    UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert oracle.rel_err(uh[[0, 1]], UB[[0, 1]]) <= BF16_GATE


@pytest.mark.parametrize("udt", ["fp32", "fp16"])
def test_commit_verify_pseudo_values_short_paths_and_faults(gpu_lib, udt):
    """max_path 13 (the first 32-slot chunk holds every path): a clean
    sequence, an out-of-range id, a path longer than max_path, an empty path;
    faulted and empty paths leave the state bit-unchanged"""
    rng = np.random.default_rng(41)
    pprev = np.stack([gs.random_recursive_tree(rng, 64, max_depth=12) for _ in range(4)])
    pcur = np.stack([gs.random_recursive_tree(rng, 64, max_depth=12) for _ in range(4)])
    acc = np.array([gs.pick_leaf(rng, pprev[i]) for i in range(4)], np.int32)
    A = gs.make_set(pprev, 2, 128, 128, "bf16", seed=41, accepted=acc)
    B = gs.make_set(pcur, 2, 128, 128, "bf16", seed=42)
    dA, dB = upload(A), upload(B)
    S = dA["S0"].clone()
    prevA = (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"])
    uA = torch.empty(dA["v"].shape, dtype=U_DTYPES[udt], device="cuda")
    uB = torch.empty(dB["v"].shape, dtype=U_DTYPES[udt], device="cuda")
    path, plen = A.paths(max_path=13)
    gpu_lib.commit_verify(S, dev(path), dev(np.zeros(4, np.int32)), prevA, dA["q"], dA["k"],
                          dA["v"], dA["alpha"], dA["beta"], dA["parent"], u_out=uA)
    path[1, 0] = 70                     # sequence 1: id out of range
    plen[2] = 14                        # sequence 2: longer than max_path
    plen[3] = 0                         # sequence 3: nothing to commit
    st = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    outB = gpu_lib.commit_verify(S, dev(path), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                                 dB["alpha"], dB["beta"], dB["parent"], u_prev=uA, u_out=uB,
                                 status=st)
    torch.cuda.synchronize()
    oref, Sref, rst = oracle_commit_verify(A, B, path, plen)
    assert host(st).tolist() == rst.tolist() == [0, 2, 2, 0]
    Sh, oh, uh = host(S), host(outB), host(uB)
    for b in (1, 2, 3):
        assert np.array_equal(Sh[b], A.S0[b]), b
    assert oracle.rel_err(Sh[0], Sref[0]) <= BF16_GATE
    assert oracle.rel_err(oh, oref) <= BF16_GATE
    UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert oracle.rel_err(uh, UB) <= BF16_GATE


# ---------------------------------------------------------------------------
# width-w best-first tree construction: bit-exact (fp32 score order)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("batch,n,K,w,md", [(16, 64, 8, 8, 12), (4, 128, 32, 16, 16),
                                            (3, 40, 5, 1, 6), (2, 126, 8, 8, 16),
                                            (5, 64, 3, 64, 2), (1, 1, 4, 2, 3)])
def test_tree_build_bit_exact(gpu_lib, batch, n, K, w, md):
    say("tree build", batch, n, K, w, md)
    lp, tok, root = gs.candidate_table(np.random.default_rng(n + K + w), batch, n, K)
    if batch > 1:
        lp[1, 3, :] = np.nan            # a node with no candidates
    par, tk, sc, nb = gpu_lib.build_tree(dev(lp), dev(tok), dev(root), w, md)
    torch.cuda.synchronize()
    rp, rt, rs, rn = oracle.build_trees(lp, tok, root, w, md)
    assert np.array_equal(host(nb), rn)
    assert np.array_equal(host(par), rp) and np.array_equal(host(tk), rt)
    assert np.array_equal(host(sc).view(np.uint32), rs.view(np.uint32))


def test_tree_build_ties_and_dry(gpu_lib):
    lp = np.zeros((2, 20, 4), np.float32)   # every score ties: the order alone decides
    lp[:, :, 3] = -np.inf
    lp[1, 1:, :] = -np.inf                  # sequence 1 runs dry after the root's children
    tok = np.arange(2 * 20 * 4, dtype=np.int32).reshape(2, 20, 4)
    par, tk, sc, nb = gpu_lib.build_tree(dev(lp), dev(tok), None, 3, 20)
    torch.cuda.synchronize()
    rp, rt, rs, rn = oracle.build_trees(lp, tok, np.full(2, -1, np.int32), 3, 20)
    assert host(nb).tolist() == rn.tolist() == [20, 4]
    assert np.array_equal(host(par), rp) and np.array_equal(host(tk), rt)
    assert np.array_equal(host(sc).view(np.uint32), rs.view(np.uint32))


def test_tree_build_hand_worked_ties(gpu_lib):
    """the hand-derived tie cases (tests/golden/tree_build_ties.json), each
    case its own launch: every ordering decision is a tie"""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "tree_build_ties.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        say("tie case", c["name"])
        lp = np.array([[-np.inf if x is None else x for x in row] for row in c["cand_logp"]],
                      np.float32)[None]
        ii, jj = np.meshgrid(np.arange(lp.shape[1]), np.arange(lp.shape[2]), indexing="ij")
        tok = np.where(np.isfinite(lp[0]), 100 + 10 * ii + jj, -1).astype(np.int32)[None]
        root = np.array([c["root_tok"]], np.int32)
        par, tk, sc, nb = gpu_lib.build_tree(dev(lp), dev(tok), dev(root), c["width"],
                                             c["max_depth"])
        torch.cuda.synchronize()
        want = np.array([-np.inf if x is None else x for x in c["score"]], np.float32)
        assert host(nb).tolist() == [c["n_built"]]
        assert host(par)[0].tolist() == c["parent"]
        assert host(tk)[0].tolist() == c["token"]
        assert np.array_equal(host(sc)[0].view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("K,w", [(8, 4), (8, 1), (16, 8), (32, 3)])
def test_tree_build_rounding_ties(gpu_lib, K, w):
    """log-probs near -8 that differ by less than a unit in the last place of
    the running scores (|score| 16..128): many pairs of one row round to the
    same fp32 score although their log-probs differ, in random slot order;
    such ties pop by slot, so the order of the raw log-probs must not
    decide.  Bit-exact against the oracle."""
    rng = np.random.default_rng(K * 10 + w)
    batch, n = 6, 48
    base = -8.0 + 0.5 * rng.integers(0, 3, size=(batch, n, K))
    lp = (base + rng.uniform(-3e-7, 3e-7, size=base.shape)).astype(np.float32)
    lp[rng.random(lp.shape) < 0.15] = -np.inf
    lp[:, 0, 0] = -8.0                       # the root proposes something
    tok = rng.integers(0, 50000, size=lp.shape).astype(np.int32)
    root = rng.integers(0, 50000, size=batch).astype(np.int32)
    par, tk, sc, nb = gpu_lib.build_tree(dev(lp), dev(tok), dev(root), w, 16)
    torch.cuda.synchronize()
    rp, rt, rs, rn = oracle.build_trees(lp, tok, root, w, 16)
    assert host(nb).tolist() == rn.tolist()
    assert np.array_equal(host(par), rp) and np.array_equal(host(tk), rt)
    assert np.array_equal(host(sc).view(np.uint32), rs.view(np.uint32))


def test_tree_build_overflowing_scores(gpu_lib):
    # scores that overflow to -inf are still candidates (popped last, by push
    # order), and a +inf score is popped first
    lp = np.full((2, 12, 3), -3e38, np.float32)
    lp[1, 0, 1] = np.float32(3e38)
    lp[1, 1, 0] = np.float32(3e38)           # node 1 (3e38) proposes +inf
    tok = np.arange(2 * 12 * 3, dtype=np.int32).reshape(2, 12, 3)
    root = np.array([5, 6], np.int32)
    par, tk, sc, nb = gpu_lib.build_tree(dev(lp), dev(tok), dev(root), 2, 6)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):
        rp, rt, rs, rn = oracle.build_trees(lp, tok, root, 2, 6)
    assert np.isneginf(rs).any() and np.isposinf(rs).any()
    assert np.array_equal(host(nb), rn)
    assert np.array_equal(host(par), rp) and np.array_equal(host(tk), rt)
    assert np.array_equal(host(sc).view(np.uint32), rs.view(np.uint32))


# ---------------------------------------------------------------------------
# greedy acceptance walk: bit-exact, then path + fused step from it
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_accept_bit_exact(gpu_lib, cfg):
    ts = gs.make_config(cfg)
    rng = np.random.default_rng(cfg)
    draft, verify = gs.make_accept_tokens(rng, ts.parent, p_match=0.8)
    st = torch.full((ts.parent.shape[0],), -7, dtype=torch.int32, device="cuda")
    acc, alen, bonus = gpu_lib.accept(dev(ts.parent), dev(draft), dev(verify), status=st)
    torch.cuda.synchronize()
    ra, rl, rb, rs = oracle.accept(ts.parent, draft, verify)
    assert np.array_equal(host(acc), ra) and np.array_equal(host(alen), rl)
    assert np.array_equal(host(bonus), rb) and np.array_equal(host(st), rs)


def test_accept_ties_and_faults_on_gpu(gpu_lib):
    rng = np.random.default_rng(9)
    par = np.stack([gs.random_recursive_tree(rng, 100) for _ in range(6)])
    draft = rng.integers(0, 3, size=par.shape).astype(np.int32)    # many sibling ties
    verify = rng.integers(0, 3, size=par.shape).astype(np.int32)
    par[2, 50] = 70
    par[4, 0] = 0
    st = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    acc, alen, bonus = gpu_lib.accept(dev(par), dev(draft), dev(verify), status=st)
    torch.cuda.synchronize()
    ra, rl, rb, rs = oracle.accept(par, draft, verify)
    assert np.array_equal(host(acc), ra) and np.array_equal(host(alen), rl)
    assert np.array_equal(host(bonus), rb) and np.array_equal(host(st), rs)
    assert rs.tolist() == [0, 0, 1, 0, 1, 0]


def test_accept_then_path_then_fused_step(gpu_lib):
    """the decode-loop order: accept on the verified tree, extract the path,
    commit it fused with the next tree's verify"""
    prev, cur = gs.make_config(2, s=3), gs.make_config(2, s=4)
    rng = np.random.default_rng(4)
    draft, verify = gs.make_accept_tokens(rng, prev.parent, p_match=0.8)
    dpar = dev(prev.parent)
    acc, _, _ = gpu_lib.accept(dpar, dev(draft), dev(verify))
    p, pl = gpu_lib.path(dpar, acc, 13)
    ra, _, _, _ = oracle.accept(prev.parent, draft, verify)
    rp, rpl, _ = oracle.path(prev.parent, ra, 13)
    assert np.array_equal(host(p), rp) and np.array_equal(host(pl), rpl)
    out, S, st = run_commit_verify(gpu_lib, prev, cur, rp, rpl)
    oref, Sref, rst = oracle_commit_verify(prev, cur, rp, rpl)
    assert st.tolist() == rst.tolist() == [0] * 16
    assert oracle.rel_err(S, Sref) <= BF16_GATE and oracle.rel_err(out, oref) <= BF16_GATE


# ---------------------------------------------------------------------------
# integer work: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_index_and_path_bit_exact(gpu_lib, cfg):
    ts = gs.make_config(cfg)
    par = ts.parent
    depth, anc = gpu_lib.index(dev(par))
    rd, ra, rs = oracle.index(par)
    assert np.array_equal(host(depth), rd)
    assert np.array_equal(host(anc).view(np.uint32), ra)
    for mp in (1, 5, 13, par.shape[1]):
        st = torch.full((par.shape[0],), -7, dtype=torch.int32, device="cuda")
        p, pl = gpu_lib.path(dev(par), dev(ts.accepted), mp, status=st)
        rp, rpl, rps = oracle.path(par, ts.accepted, mp)
        assert np.array_equal(host(p), rp) and np.array_equal(host(pl), rpl)
        assert np.array_equal(host(st), rps)


def test_index_and_path_malformed(gpu_lib):
    rng = np.random.default_rng(4)
    par = np.stack([gs.random_recursive_tree(rng, 77) for _ in range(8)])
    par[1, 76] = 76
    par[2, 5] = -4
    par[3, 40] = 50
    acc = rng.integers(0, 77, size=8).astype(np.int32)
    acc[1], acc[4], acc[5] = 76, 77, -1
    st = torch.full((8,), -7, dtype=torch.int32, device="cuda")
    depth, anc = gpu_lib.index(dev(par), status=st)
    rd, ra, rs = oracle.index(par)
    assert np.array_equal(host(depth), rd) and np.array_equal(host(anc).view(np.uint32), ra)
    assert np.array_equal(host(st), rs)
    for mp in (3, 77):
        p, pl = gpu_lib.path(dev(par), dev(acc), mp, status=st)
        rp, rpl, rps = oracle.path(par, acc, mp)
        assert np.array_equal(host(p), rp) and np.array_equal(host(pl), rpl)
        assert np.array_equal(host(st), rps)
