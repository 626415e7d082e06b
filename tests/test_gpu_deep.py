"""GPU parity on deep and wide trees, and on whole workload tensors.

The 64-node kernels (gdn_tree_verify for n <= 64 and the fused
gdn_tree_commit_verify) on the tree shapes that stress them most: chains of
64, 63 and 33 nodes (the last pointer-jumping rounds of the topology, and a
dense coupling block X_10 between the two 32-row halves of the solve), a
64-node star, an 8-ary breadth-first bush and a two-root forest.  The
method is the DFlash-TfM page's rollback-free tree verification for GDN:
the tree is topologically sorted, X and Y follow the ancestor relations,
(I + X) U = beta V (with the committed-state term) is solved without
touching the state, and the commit follows the accepted branch.

Every comparison is against the fp64 oracle over the whole output tensor:
max|gpu - ref| / max|ref| <= 2e-3 (bf16 q/k/v, fp32 state).
"""
import numpy as np
import pytest
import torch

import gdn_synth as gs
import oracle
from gpu_util import dev, host, upload

pytestmark = pytest.mark.gpu

BF16_GATE = 2e-3


def say(*a):
    print(*a, flush=True)


def forest64():
    """two roots: a 20-node chain and a random tree of 44 nodes below the
    second root (node 20)"""
    rng = np.random.default_rng(77)
    p = gs.random_recursive_tree(rng, 44, max_depth=20) + 20
    p[0] = -1
    return np.concatenate([gs.chain_tree(20), p]).astype(np.int32)


def deep_random_tree(rng, n):
    """a deep random tree: node i hangs below one of its few predecessors
    (i - g with g ~ Geometric(0.6)), so depth grows with n and side branches
    stay short"""
    p = np.full(n, -1, np.int32)
    for i in range(1, n):
        p[i] = max(0, i - int(rng.geometric(0.6)))
    return p


def deep_set_n64():
    """batch of five 64-node trees: chain, star, 8-ary bush, forest, and a
    deep random tree"""
    rng = np.random.default_rng(64)
    par = np.stack([gs.chain_tree(64), gs.star_tree(64), gs.kary_bfs_tree(64, 8), forest64(),
                    deep_random_tree(rng, 64)])
    depth = np.array([max(gs._depths(p)) for p in par])
    assert depth.tolist()[:3] == [63, 1, 2] and depth[4] > 32
    return par


# ---------------------------------------------------------------------------
# verify, n <= 64 kernel
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["n64_mixed", "chain63", "chain33", "chain32", "chain1"])
def test_verify_deep_trees_n64(gpu_lib, case):
    say("verify deep", case)
    par = {"n64_mixed": deep_set_n64(), "chain63": np.stack([gs.chain_tree(63)] * 2),
           "chain33": np.stack([gs.chain_tree(33)] * 2),
           "chain32": np.stack([gs.chain_tree(32)] * 2),
           "chain1": np.stack([gs.chain_tree(1)] * 2)}[case]
    ts = gs.make_set(par, 4, 128, 128, "bf16", seed=600 + par.shape[1])
    d = upload(ts)
    st = torch.full((par.shape[0],), -7, dtype=torch.int32, device="cuda")
    out = gpu_lib.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"],
                         status=st)
    torch.cuda.synchronize()
    ref, rst = oracle.verify_set(ts)
    assert host(st).tolist() == rst.tolist() == [0] * par.shape[0]
    err = oracle.rel_err(host(out), ref)
    say("rel err", err)
    assert err <= BF16_GATE
    for b in range(par.shape[0]):
        assert oracle.rel_err(host(out)[b], ref[b]) <= BF16_GATE, b


# ---------------------------------------------------------------------------
# fused commit + verify on the same shapes, both commit modes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["solving", "carried_fp32", "carried_fp16"])
def test_commit_verify_deep_trees_n64(gpu_lib, mode):
    """call 1 verifies tree set A (no commit) and, for the carried modes,
    writes its pseudo-values; call 2 commits each sequence's accepted branch
    of A (a 64-node path on the chain, deep branches elsewhere) and verifies
    tree set B.  Both calls' outputs, the pseudo-values and the committed
    state against the oracle, whole tensors."""
    say("commit-verify deep", mode)
    pa = deep_set_n64()
    pb = deep_set_n64()[::-1].copy()
    acc = np.array([63, 17, 63, 19, 0], np.int32)
    acc[4] = int(np.argmax(gs._depths(pa[4])))          # the deepest node
    A = gs.make_set(pa, 4, 128, 128, "bf16", seed=611, accepted=acc)
    B = gs.make_set(pb, 4, 128, 128, "bf16", seed=612)
    dA, dB = upload(A), upload(B)
    path, plen = A.paths(max_path=64)
    assert plen.tolist()[:4] == [64, 2, 3, 20]
    udt = {"solving": None, "carried_fp32": torch.float32, "carried_fp16": torch.float16}[mode]
    uA = uB = None
    if udt is not None:
        uA = torch.empty(dA["v"].shape, dtype=udt, device="cuda")
        uB = torch.empty(dB["v"].shape, dtype=udt, device="cuda")
    S = dA["S0"].clone()
    prevA = (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"])
    st = torch.full((5,), -7, dtype=torch.int32, device="cuda")
    outA = gpu_lib.commit_verify(S, dev(path), dev(np.zeros(5, np.int32)), prevA, dA["q"],
                                 dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"],
                                 u_out=uA, status=st)
    torch.cuda.synchronize()
    refA, _ = oracle.verify_set(A)
    assert host(st).tolist() == [0] * 5 and torch.equal(S, dA["S0"])
    eA = oracle.rel_err(host(outA), refA)
    say("call 1 out rel err", eA)
    assert eA <= BF16_GATE
    if uA is not None:
        UA, _ = oracle.pseudo_set(A)
        eu = oracle.rel_err(host(uA), UA)
        say("call 1 u rel err", eu)
        assert eu <= BF16_GATE
    outB = gpu_lib.commit_verify(S, dev(path), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                                 dB["alpha"], dB["beta"], dB["parent"], u_prev=uA, u_out=uB,
                                 status=st)
    torch.cuda.synchronize()
    Sref, cst = oracle.commit_set(A, path_arr=path, path_len=plen)
    oref, vst = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert host(st).tolist() == (cst | vst).tolist() == [0] * 5
    es, eo = oracle.rel_err(host(S), Sref), oracle.rel_err(host(outB), oref)
    say("call 2 rel err S", es, "out", eo)
    assert es <= BF16_GATE and eo <= BF16_GATE
    for b in range(5):
        assert oracle.rel_err(host(S)[b], Sref[b]) <= BF16_GATE, b
        assert oracle.rel_err(host(outB)[b], oref[b]) <= BF16_GATE, b
    if uB is not None:
        UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
        assert oracle.rel_err(host(uB), UB) <= BF16_GATE


@pytest.mark.parametrize("n", [32, 17, 1])
@pytest.mark.parametrize("batch", [1, 8])
def test_verify_small_trees_both_launch_shapes(gpu_lib, n, batch):
    """gdn_tree_verify on trees of at most 32 nodes with 32 heads: batch 1
    takes the d_v-split launch (four single-wave workgroups per sequence and
    head, each forming the tree matrices itself and solving a quarter of the
    d_v columns), batch 8 the one-block instance of the 64-node kernel (one
    workgroup per sequence and head); chains, stars, random trees and
    two-root forests, whole tensors against the oracle"""
    say("verify small trees", n, batch)
    rng = np.random.default_rng(31 * n + batch)
    shapes = [gs.chain_tree(n), gs.star_tree(n), gs.random_recursive_tree(rng, n, 8)]
    if n >= 4:
        f = gs.random_recursive_tree(rng, n, 6)
        f[n // 2] = -1                     # a second root
        shapes.append(f)
    par = np.stack([shapes[b % len(shapes)] for b in range(batch)])
    ts = gs.make_set(par, 32, 128, 128, "bf16", seed=900 + n + batch)
    d = upload(ts)
    st = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    out = gpu_lib.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"],
                         status=st)
    torch.cuda.synchronize()
    ref, rst = oracle.verify_set(ts)
    assert host(st).tolist() == rst.tolist() == [0] * batch
    for b in range(batch):
        err = oracle.rel_err(host(out)[b], ref[b])
        say("seq", b, "rel err", err)
        assert err <= BF16_GATE, b
    assert torch.equal(d["S0"], upload(ts)["S0"])   # the state is only read


def test_verify_split_launch_bad_parent(gpu_lib):
    """the d_v-split launch on a malformed tree: that sequence's output rows
    are NaN in every quarter, its status flag is set once, the other
    sequence is verified as usual"""
    rng = np.random.default_rng(5)
    par = np.stack([gs.random_recursive_tree(rng, 32, 8) for _ in range(2)])
    par[1, 5] = 5                          # a node that is its own parent
    ts = gs.make_set(par, 32, 128, 128, "bf16", seed=905)
    d = upload(ts)
    st = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    out = host(gpu_lib.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                              d["S0"], status=st))
    ref, rst = oracle.verify_set(ts)
    assert host(st).tolist() == rst.tolist() == [0, 1]
    assert np.isnan(out[1]).all() and np.isfinite(out[0]).all()
    assert oracle.rel_err(out[0], ref[0]) <= BF16_GATE


@pytest.mark.parametrize("n", [32, 17, 1])
@pytest.mark.parametrize("max_path", [16, 32])
@pytest.mark.parametrize("mode", ["solving", "carried_fp32", "carried_fp16"])
def test_commit_verify_one_block_trees(gpu_lib, n, max_path, mode):
    """new trees of at most 32 nodes (the kernels' one-block instances: only
    the first 32-row block contracted and solved) after previous 32-node
    trees: call 1 verifies set A, call 2 commits A's accepted branches (a
    32-node path on the chain when max_path allows it) and verifies set B;
    outputs, pseudo-values and the committed state against the oracle"""
    say("commit-verify one block", n, max_path, mode)
    rng = np.random.default_rng(n + 7 * max_path)
    pa = np.stack([gs.chain_tree(32), gs.star_tree(32), gs.random_recursive_tree(rng, 32, 8)])
    pb = np.stack([gs.chain_tree(n), gs.star_tree(n), gs.random_recursive_tree(rng, n, 8)])
    acc = np.array([min(31, max_path - 1), 9, int(np.argmax(gs._depths(pa[2])))], np.int32)
    A = gs.make_set(pa, 4, 128, 128, "bf16", seed=700 + max_path, accepted=acc)
    B = gs.make_set(pb, 4, 128, 128, "bf16", seed=701 + n)
    dA, dB = upload(A), upload(B)
    path, plen = A.paths(max_path=max_path)
    udt = {"solving": None, "carried_fp32": torch.float32, "carried_fp16": torch.float16}[mode]
    uA = uB = None
    if udt is not None:
        uA = torch.empty(dA["v"].shape, dtype=udt, device="cuda")
        uB = torch.empty(dB["v"].shape, dtype=udt, device="cuda")
    S = dA["S0"].clone()
    prevA = (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"])
    st = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    outA = gpu_lib.commit_verify(S, dev(path), dev(np.zeros(3, np.int32)), prevA, dA["q"],
                                 dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"],
                                 u_out=uA, status=st)
    torch.cuda.synchronize()
    refA, _ = oracle.verify_set(A)
    assert host(st).tolist() == [0] * 3 and torch.equal(S, dA["S0"])
    assert oracle.rel_err(host(outA), refA) <= BF16_GATE
    outB = gpu_lib.commit_verify(S, dev(path), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                                 dB["alpha"], dB["beta"], dB["parent"], u_prev=uA, u_out=uB,
                                 status=st)
    torch.cuda.synchronize()
    Sref, cst = oracle.commit_set(A, path_arr=path, path_len=plen)
    oref, vst = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert host(st).tolist() == (cst | vst).tolist() == [0] * 3
    es, eo = oracle.rel_err(host(S), Sref), oracle.rel_err(host(outB), oref)
    say("rel err S", es, "out", eo)
    assert es <= BF16_GATE and eo <= BF16_GATE
    for b in range(3):
        assert oracle.rel_err(host(S)[b], Sref[b]) <= BF16_GATE, b
        assert oracle.rel_err(host(outB)[b], oref[b]) <= BF16_GATE, b
    if uB is not None:
        UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
        assert oracle.rel_err(host(uB), UB) <= BF16_GATE


@pytest.mark.parametrize("n", [32, 17, 1])
@pytest.mark.parametrize("mode", ["solving", "carried_fp32", "carried_fp16"])
def test_commit_verify_split_launch(gpu_lib, n, mode):
    """the d_v-split fused launch (2 sequences x 32 heads: four three-wave
    workgroups per sequence and head, each committing and verifying a
    quarter of the d_v columns): call 1 verifies the 32-node trees A and
    writes their pseudo-values, call 2 commits A's accepted branches (16
    nodes for the solving commit, 32 with pseudo-values carried) and
    verifies the trees B; then a call with a malformed new tree on
    sequence 0 (its branch still committed, NaN outputs) and an id out of
    range on sequence 1's path (state unchanged)"""
    say("commit-verify split launch", n, mode)
    rng = np.random.default_rng(n + 17)
    max_path = 16 if mode == "solving" else 32
    pa = np.stack([gs.random_recursive_tree(rng, 32, 8), gs.chain_tree(32)])
    pb = np.stack([gs.chain_tree(n), gs.random_recursive_tree(rng, n, 8)])
    acc = np.array([int(np.argmax(gs._depths(pa[0]))), max_path - 1], np.int32)
    A = gs.make_set(pa, 32, 128, 128, "bf16", seed=760 + n, accepted=acc)
    B = gs.make_set(pb, 32, 128, 128, "bf16", seed=761 + n)
    dA, dB = upload(A), upload(B)
    path, plen = A.paths(max_path=max_path)
    udt = {"solving": None, "carried_fp32": torch.float32, "carried_fp16": torch.float16}[mode]
    uA = uB = None
    if udt is not None:
        uA = torch.empty(dA["v"].shape, dtype=udt, device="cuda")
        uB = torch.empty(dB["v"].shape, dtype=udt, device="cuda")
    S = dA["S0"].clone()
    prevA = (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"])
    st = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    outA = gpu_lib.commit_verify(S, dev(path), dev(np.zeros(2, np.int32)), prevA, dA["q"],
                                 dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"],
                                 u_out=uA, status=st)
    torch.cuda.synchronize()
    refA, _ = oracle.verify_set(A)
    assert host(st).tolist() == [0, 0] and torch.equal(S, dA["S0"])
    assert oracle.rel_err(host(outA), refA) <= BF16_GATE
    if uA is not None:
        UA, _ = oracle.pseudo(A.k, A.v, A.alpha, A.beta, A.parent, A.S0)
        assert oracle.rel_err(host(uA), UA) <= BF16_GATE
    outB = gpu_lib.commit_verify(S, dev(path), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                                 dB["alpha"], dB["beta"], dB["parent"], u_prev=uA, u_out=uB,
                                 status=st)
    torch.cuda.synchronize()
    Sref, cst = oracle.commit_set(A, path_arr=path, path_len=plen)
    oref, vst = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert host(st).tolist() == (cst | vst).tolist() == [0, 0]
    for b in range(2):
        assert oracle.rel_err(host(S)[b], Sref[b]) <= BF16_GATE, b
        assert oracle.rel_err(host(outB)[b], oref[b]) <= BF16_GATE, b
    if uB is not None:
        UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
        assert oracle.rel_err(host(uB), UB) <= BF16_GATE
    # faults: sequence 0's new tree malformed, sequence 1's path out of range
    S = dA["S0"].clone()
    badB = B.parent.copy()
    badB[0, 0] = -5
    bpath = path.copy()
    bpath[1, plen[1] - 1] = 32
    outF = gpu_lib.commit_verify(S, dev(bpath), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                                 dB["alpha"], dB["beta"], dev(badB), u_prev=uA, u_out=uB,
                                 status=st)
    torch.cuda.synchronize()
    assert host(st).tolist() == [1, 2]
    assert oracle.rel_err(host(S)[0], Sref[0]) <= BF16_GATE
    assert np.array_equal(host(S)[1], A.S0[1])
    assert np.isnan(host(outF)[0]).all()
    if uB is not None:
        assert np.isnan(host(uB)[0].astype(np.float32)).all()
    o1, _ = oracle.verify(B.q[1:], B.k[1:], B.v[1:], B.alpha[1:], B.beta[1:], B.parent[1:],
                          A.S0[1:])
    assert oracle.rel_err(host(outF)[1], o1[0]) <= BF16_GATE


@pytest.mark.parametrize("n", [128, 32, 16])
def test_commit_split_launch(gpu_lib, n):
    """gdn_tree_commit on a small launch (2 sequences x 32 heads: four
    two-wave workgroups per sequence and head, each committing a quarter of
    the d_v columns) with paths of up to 16 nodes: a chain's first 16 nodes
    (the whole chunk) and a random tree's deepest path; then the same with
    an id out of range on sequence 1 (state unchanged) and an empty path on
    sequence 0 (a no-op)"""
    say("commit split launch", n)
    rng = np.random.default_rng(n + 3)
    par = np.stack([gs.chain_tree(n), gs.random_recursive_tree(rng, n, 12)])
    d1 = gs._depths(par[1])
    leaf = int(np.argmax(np.where(d1 < 16, d1, -1)))
    ts = gs.make_set(par, 32, 128, 128, "bf16", seed=880 + n,
                     accepted=np.array([15, leaf], np.int32))
    d = upload(ts)
    path, plen = ts.paths(max_path=16)
    assert plen.tolist() == [16, int(d1[leaf]) + 1]
    S = d["S0"].clone()
    st = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    gpu_lib.commit(S, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                   status=st)
    torch.cuda.synchronize()
    Sref, rst = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert host(st).tolist() == rst.tolist() == [0, 0]
    for b in range(2):
        assert oracle.rel_err(host(S)[b], Sref[b]) <= BF16_GATE, b
    bpath, bplen = path.copy(), plen.copy()
    bplen[0] = 0
    bpath[1, bplen[1] - 1] = n
    S = d["S0"].clone()
    gpu_lib.commit(S, dev(bpath), dev(bplen), d["k"], d["v"], d["alpha"], d["beta"],
                   d["parent"], status=st)
    torch.cuda.synchronize()
    assert host(st).tolist() == [0, 2]
    assert torch.equal(S, d["S0"])


@pytest.mark.parametrize("udt", [torch.float32, torch.float16])
def test_carried_commit_rejects_a_faulted_previous_tree(gpu_lib, udt):
    """a well-formed path through a previous tree whose parent row is
    malformed elsewhere: that tree's verify wrote NaN pseudo-values, so the
    carried commit must not use them (GDN_FAULT_BAD_PATH, state unchanged);
    the solving commit, which needs only the path, commits it"""
    rng = np.random.default_rng(71)
    pa = np.stack([gs.random_recursive_tree(rng, 48, max_depth=10) for _ in range(3)])
    acc = np.array([gs.pick_leaf(rng, pa[i]) for i in range(3)], np.int32)
    path_nodes = set(gs.path_to(pa[1], int(acc[1])).tolist())
    bad = max(i for i in range(1, 48) if i not in path_nodes)
    pa[1, bad] = bad                       # sequence 1: malformed, off its path
    A = gs.make_set(pa, 2, 128, 128, "bf16", seed=71, accepted=acc)
    B = gs.make_set(np.stack([gs.random_recursive_tree(rng, 48, max_depth=10)
                              for _ in range(3)]), 2, 128, 128, "bf16", seed=72)
    dA, dB = upload(A), upload(B)
    prevA = (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"])
    path, plen = A.paths(max_path=13)
    uA = torch.empty(dA["v"].shape, dtype=udt, device="cuda")
    S = dA["S0"].clone()
    st = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    gpu_lib.commit_verify(S, dev(path), dev(np.zeros(3, np.int32)), prevA, dA["q"], dA["k"],
                          dA["v"], dA["alpha"], dA["beta"], dA["parent"], u_out=uA, status=st)
    torch.cuda.synchronize()
    assert host(st).tolist() == [0, 1, 0]
    assert np.isnan(host(uA)[1]).all()
    Sref, cst = oracle.commit_set(A, path_arr=path, path_len=plen)
    assert cst.tolist() == [0, 0, 0]       # the path alone is valid
    oref_moved, _ = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    oref_kept, _ = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, A.S0)
    # carried: sequence 1 keeps its state
    out = gpu_lib.commit_verify(S, dev(path), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                                dB["alpha"], dB["beta"], dB["parent"], u_prev=uA, status=st)
    torch.cuda.synchronize()
    assert host(st).tolist() == [0, 2, 0]
    Sh, oh = host(S), host(out)
    assert np.array_equal(Sh[1], A.S0[1]) and not np.isnan(Sh).any()
    assert oracle.rel_err(Sh[[0, 2]], Sref[[0, 2]]) <= BF16_GATE
    assert oracle.rel_err(oh[1], oref_kept[1]) <= BF16_GATE
    assert oracle.rel_err(oh[[0, 2]], oref_moved[[0, 2]]) <= BF16_GATE
    # solving: every path is committed
    S2 = dA["S0"].clone()
    gpu_lib.commit_verify(S2, dev(path), dev(plen), prevA, dB["q"], dB["k"], dB["v"],
                          dB["alpha"], dB["beta"], dB["parent"], status=st)
    torch.cuda.synchronize()
    assert host(st).tolist() == [0, 0, 0]
    assert oracle.rel_err(host(S2), Sref) <= BF16_GATE


# ---------------------------------------------------------------------------
# whole workload tensors
# ---------------------------------------------------------------------------
def test_verify_layer_b64_n128_full(gpu_lib):
    """the batch-64, 128-node workload (a quarter chains, a quarter stars and
    16-ary bushes, half random recursive trees), whole output tensor, and the
    commit of every sequence's accepted branch, whole state"""
    say("verify b64 n128 full")
    ts = gs.make_config(3)
    d = upload(ts)
    st = torch.full((64,), -7, dtype=torch.int32, device="cuda")
    out = gpu_lib.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"],
                         status=st)
    path, plen = ts.paths(max_path=128)
    S = d["S0"].clone()
    gpu_lib.commit(S, dev(path), dev(plen), d["k"], d["v"], d["alpha"], d["beta"], d["parent"])
    torch.cuda.synchronize()
    ref, rst = oracle.verify_set(ts)
    assert host(st).tolist() == rst.tolist() == [0] * 64
    err = oracle.rel_err(host(out), ref)
    say("verify rel err", err)
    assert err <= BF16_GATE
    for b in range(64):
        assert oracle.rel_err(host(out)[b], ref[b]) <= BF16_GATE, b
    Sref, _ = oracle.commit_set(ts, path_arr=path, path_len=plen)
    es = oracle.rel_err(host(S), Sref)
    say("commit rel err", es)
    assert es <= BF16_GATE


def test_commit_verify_b64_n128_full(gpu_lib):
    """the batch-64, 128-node workload as one fused step (two workgroups per
    CU, 2048 of them: the commit of set 0's accepted branches, then set 1's
    trees verified from the committed state, with the new pseudo-values
    out): whole state, output and pseudo-value tensors against the oracle"""
    say("commit-verify b64 n128 full")
    A, B = gs.make_config(3, s=0), gs.make_config(3, s=1)
    dA, dB = upload(A), upload(B)
    path, plen = A.paths(max_path=128)
    S = dA["S0"].clone()
    u = torch.empty(dB["v"].shape, dtype=torch.float32, device="cuda")
    st = torch.full((64,), -7, dtype=torch.int32, device="cuda")
    out = gpu_lib.commit_verify(S, dev(path), dev(plen),
                                (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"]),
                                dB["q"], dB["k"], dB["v"], dB["alpha"], dB["beta"], dB["parent"],
                                u_out=u, status=st)
    torch.cuda.synchronize()
    Sref, cst = oracle.commit_set(A, path_arr=path, path_len=plen)
    oref, vst = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert host(st).tolist() == (cst | vst).tolist() == [0] * 64
    es, eo = oracle.rel_err(host(S), Sref), oracle.rel_err(host(out), oref)
    say("rel err S", es, "out", eo)
    assert es <= BF16_GATE and eo <= BF16_GATE
    for b in range(64):
        assert oracle.rel_err(host(S)[b], Sref[b]) <= BF16_GATE, b
        assert oracle.rel_err(host(out)[b], oref[b]) <= BF16_GATE, b
    UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    eu = oracle.rel_err(host(u), UB)
    say("u rel err", eu)
    assert eu <= BF16_GATE


def test_stack48_layers_from_the_stacked_run(gpu_lib):
    """the 48-layer stack (batch 32, 32 heads, one 64-node tree per sequence
    shared by all layers): per-layer tensors stacked in one allocation each,
    every layer's decode step run in layer order (a fused call verifying the
    tree from the layer's state and writing its pseudo-values, then a fused
    call committing the accepted branch from them and verifying the tree
    again); layers 0 and 47 hold the workload's seeded tensors and are
    checked whole against the oracle, the other layers hold other random
    values."""
    say("stack48 stacked run")
    L = 48
    t0, t47 = gs.make_config(4, layer=0), gs.make_config(4, layer=47)
    assert np.array_equal(t0.parent, t47.parent)
    d0, d47 = upload(t0), upload(t47)
    gen = torch.Generator(device="cuda").manual_seed(4)

    def stack(key, fill):
        x = torch.empty((L,) + tuple(d0[key].shape), dtype=d0[key].dtype, device="cuda")
        x[0], x[L - 1] = d0[key], d47[key]
        for l in range(1, L - 1):
            x[l] = fill(x[l].shape)
        return x

    nrm = lambda s: torch.nn.functional.normalize(
        torch.randn(s, generator=gen, device="cuda"), dim=-1).to(torch.bfloat16)
    q, k = stack("q", nrm), stack("k", nrm)
    v = stack("v", lambda s: torch.randn(s, generator=gen, device="cuda").to(torch.bfloat16))
    uni = lambda s: torch.rand(s, generator=gen, device="cuda") * 0.98 + 0.01
    alpha, beta = stack("alpha", uni), stack("beta", uni)
    S = stack("S0", lambda s: torch.randn(s, generator=gen, device="cuda") / 128 ** 0.5)
    S0_47 = S[L - 1].clone()
    parent = d0["parent"]
    path, plen = t0.paths(max_path=13)
    dpath, dplen, zero = dev(path), dev(plen), dev(np.zeros(32, np.int32))
    out1 = torch.empty_like(v, dtype=torch.float32)
    out2 = torch.empty_like(out1)
    u = torch.empty_like(out1)
    st = torch.full((L, 32), -7, dtype=torch.int32, device="cuda")
    for l in range(L):
        prev = (k[l], v[l], alpha[l], beta[l], parent)
        gpu_lib.commit_verify(S[l], dpath, zero, prev, q[l], k[l], v[l], alpha[l], beta[l],
                              parent, out=out1[l], u_out=u[l], status=st[l])
    for l in range(L):
        prev = (k[l], v[l], alpha[l], beta[l], parent)
        gpu_lib.commit_verify(S[l], dpath, dplen, prev, q[l], k[l], v[l], alpha[l], beta[l],
                              parent, out=out2[l], u_prev=u[l], status=st[l])
    torch.cuda.synchronize()
    assert host(st).tolist() == [[0] * 32] * L
    for l, ts in ((0, t0), (L - 1, t47)):
        ref1, _ = oracle.verify_set(ts)
        Sref, _ = oracle.commit_set(ts, path_arr=path, path_len=plen)
        ref2, _ = oracle.verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, Sref)
        e1 = oracle.rel_err(host(out1[l]), ref1)
        es = oracle.rel_err(host(S[l]), Sref)
        e2 = oracle.rel_err(host(out2[l]), ref2)
        say("layer", l, "rel err verify", e1, "commit", es, "verify after commit", e2)
        assert e1 <= BF16_GATE and es <= BF16_GATE and e2 <= BF16_GATE
    assert not torch.equal(S[L - 1], S0_47)


# ---------------------------------------------------------------------------
# fused commit + verify for 65..128-node trees: one launch
# ---------------------------------------------------------------------------
def prev_set_n128(max_path):
    """previous trees of 128 nodes (chain, star, 16-ary bush, random of depth
    <= 16) and accepted nodes whose paths fit max_path"""
    rng = np.random.default_rng(128)
    par = np.stack([gs.chain_tree(128), gs.star_tree(128), gs.kary_bfs_tree(128, 16),
                    gs.random_recursive_tree(rng, 128, max_depth=16)])
    d3 = gs._depths(par[3])
    acc = np.array([min(127, max_path - 1), 5, 127,
                    int(np.argmax(np.where(d3 < max_path, d3, -1)))], np.int32)
    return par, acc


@pytest.mark.parametrize("n", [128, 65])
@pytest.mark.parametrize("max_path", [16, 128])
@pytest.mark.parametrize("udt", [None, torch.float32, torch.float16])
def test_commit_verify_n128_one_launch(gpu_lib, n, max_path, udt):
    """the previous trees' accepted paths committed (the solving commit; a
    128-node path on the chain when max_path allows it) and 65..128-node
    trees verified in one launch, with and without the new pseudo-values:
    state, outputs and pseudo-values against the oracle, whole tensors"""
    say("commit-verify n128", n, max_path, udt)
    pa, acc = prev_set_n128(max_path)
    rng = np.random.default_rng(n + max_path)
    pb = np.stack([gs.star_tree(n), gs.chain_tree(n), gs.random_recursive_tree(rng, n, 16),
                   gs.kary_bfs_tree(n, 8)])
    A = gs.make_set(pa, 3, 128, 128, "bf16", seed=130 + max_path, accepted=acc)
    B = gs.make_set(pb, 3, 128, 128, "bf16", seed=131 + n)
    dA, dB = upload(A), upload(B)
    path, plen = A.paths(max_path=max_path)
    assert plen.max() <= max_path and (max_path < 128 or plen[0] == 128)
    S = dA["S0"].clone()
    u = None if udt is None else torch.empty(dB["v"].shape, dtype=udt, device="cuda")
    st = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    out = gpu_lib.commit_verify(S, dev(path), dev(plen),
                                (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"]),
                                dB["q"], dB["k"], dB["v"], dB["alpha"], dB["beta"], dB["parent"],
                                u_out=u, status=st)
    torch.cuda.synchronize()
    Sref, cst = oracle.commit_set(A, path_arr=path, path_len=plen)
    oref, vst = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert host(st).tolist() == (cst | vst).tolist() == [0] * 4
    es, eo = oracle.rel_err(host(S), Sref), oracle.rel_err(host(out), oref)
    say("rel err S", es, "out", eo)
    assert es <= BF16_GATE and eo <= BF16_GATE
    for b in range(4):
        assert oracle.rel_err(host(S)[b], Sref[b]) <= BF16_GATE, b
        assert oracle.rel_err(host(out)[b], oref[b]) <= BF16_GATE, b
    if u is not None:
        UB, _ = oracle.pseudo(B.k, B.v, B.alpha, B.beta, B.parent, Sref)
        eu = oracle.rel_err(host(u), UB)
        say("u rel err", eu)
        assert eu <= BF16_GATE
        if udt == torch.float16:
            u32 = torch.empty(dB["v"].shape, dtype=torch.float32, device="cuda")
            S2 = dA["S0"].clone()
            gpu_lib.commit_verify(S2, dev(path), dev(plen),
                                  (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"]),
                                  dB["q"], dB["k"], dB["v"], dB["alpha"], dB["beta"],
                                  dB["parent"], u_out=u32)
            torch.cuda.synchronize()
            assert torch.equal(u.view(torch.int16), u32.half().view(torch.int16))


@pytest.mark.parametrize("max_path", [16, 128])
def test_commit_verify_n128_faults(gpu_lib, max_path):
    """sequence 0 clean, 1 a path with an id out of range (state bit-unchanged),
    2 a malformed new tree (NaN outputs and pseudo-values; its commit still
    applies), 3 both, 4 an empty path"""
    rng = np.random.default_rng(77 + max_path)
    pa = np.stack([gs.random_recursive_tree(rng, 128, max_depth=14) for _ in range(5)])
    pb = np.stack([gs.random_recursive_tree(rng, 96, max_depth=14) for _ in range(5)])
    acc = np.array([gs.pick_leaf(rng, pa[i]) for i in range(5)], np.int32)
    A = gs.make_set(pa, 2, 128, 128, "bf16", seed=91, accepted=acc)
    B = gs.make_set(pb, 2, 128, 128, "bf16", seed=92)
    path, plen = A.paths(max_path=max_path)
    path[1, plen[1] - 1] = 128
    path[3, 0] = 300
    plen[4] = 0
    B.parent[2, 95] = 95
    B.parent[3, 0] = -4
    dA, dB = upload(A), upload(B)
    S = dA["S0"].clone()
    u = torch.empty(dB["v"].shape, dtype=torch.float32, device="cuda")
    st = torch.full((5,), -7, dtype=torch.int32, device="cuda")
    out = gpu_lib.commit_verify(S, dev(path), dev(plen),
                                (dA["k"], dA["v"], dA["alpha"], dA["beta"], dA["parent"]),
                                dB["q"], dB["k"], dB["v"], dB["alpha"], dB["beta"], dB["parent"],
                                u_out=u, status=st)
    torch.cuda.synchronize()
    Sref, cst = oracle.commit_set(A, path_arr=path, path_len=plen)
    oref, vst = oracle.verify(B.q, B.k, B.v, B.alpha, B.beta, B.parent, Sref)
    assert host(st).tolist() == (cst | vst).tolist() == [0, 2, 1, 3, 0]
    Sh, oh, uh = host(S), host(out), host(u)
    for b in (1, 3, 4):
        assert np.array_equal(Sh[b], A.S0[b]), b
    for b in (0, 2):
        assert oracle.rel_err(Sh[b], Sref[b]) <= BF16_GATE, b
    assert np.isnan(oh[2:4]).all() and np.isnan(uh[2:4]).all()
    for b in (0, 1, 4):
        assert oracle.rel_err(oh[b], oref[b]) <= BF16_GATE, b


# ---------------------------------------------------------------------------
# more heads than the MFMA kernels' 32-bit buffer ranges take
# ---------------------------------------------------------------------------
def test_many_heads_take_the_generic_kernels(gpu_lib):
    """4097 heads (past the MFMA kernels' limit of 4096, whose byte extents
    must fit 32-bit buffer offsets): verify, commit and the fused call run
    on the generic kernels and match the oracle"""
    say("4097 heads")
    par = np.stack([np.array([-1, 0, 1, 1], np.int32)])
    prev = gs.make_set(par, 4097, 128, 128, "bf16", seed=44, accepted=np.array([3], np.int32))
    cur = gs.make_set(par, 4097, 128, 128, "bf16", seed=45)
    dp, dc = upload(prev), upload(cur)
    path, plen = prev.paths(max_path=4)
    out = gpu_lib.verify(dc["q"], dc["k"], dc["v"], dc["alpha"], dc["beta"], dc["parent"],
                         dc["S0"])
    ref, _ = oracle.verify_set(cur)
    assert oracle.rel_err(host(out), ref) <= BF16_GATE
    S = dp["S0"].clone()
    gpu_lib.commit(S, dev(path), dev(plen), dp["k"], dp["v"], dp["alpha"], dp["beta"],
                   dp["parent"])
    Sref, _ = oracle.commit_set(prev, path_arr=path, path_len=plen)
    assert oracle.rel_err(host(S), Sref) <= BF16_GATE
    S2 = dp["S0"].clone()
    out2 = gpu_lib.commit_verify(S2, dev(path), dev(plen),
                                 (dp["k"], dp["v"], dp["alpha"], dp["beta"], dp["parent"]),
                                 dc["q"], dc["k"], dc["v"], dc["alpha"], dc["beta"], dc["parent"])
    torch.cuda.synchronize()
    assert torch.equal(S2, S)
    ref2, _ = oracle.verify(cur.q, cur.k, cur.v, cur.alpha, cur.beta, cur.parent, Sref)
    assert oracle.rel_err(host(out2), ref2) <= BF16_GATE
