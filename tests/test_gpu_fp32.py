"""GPU parity of the all-fp32 fast paths (fp32 q/k/v, d_k = d_v = 128: the
fp32-MFMA verify for n <= 64 and the fp32-MFMA chunked commit) against the
fp64 oracle, at the fp32 gate max|gpu - ref| / max|ref| <= 1e-5 over whole
output and state tensors.

The method is the DFlash-TfM page's rollback-free tree verification for
GDN: the tree is topologically sorted, X and Y follow the ancestor
relations, (I + X) U = beta V (with the committed-state term) is solved
without touching the state.  Shapes: 64-node chains (the last
pointer-jumping rounds and a dense coupling block between the two 32-row
halves), a star, an 8-ary bush, a two-root forest, short chains that leave
the second block empty or ragged, the batch-16 / 32-head / 64-node layer,
malformed parents, and the fused call's fp32 fallback (commit launch, then
this verify ORing its flag into the commit's).  The commit: paths of 1 to
128 nodes (one to four 32-node chunks, full and ragged), the batch-16
layer's accepted branches, bad paths (state bit-unchanged) and an empty
path.
"""
import numpy as np
import pytest
import torch

import gdn_synth as gs
import oracle
from gpu_util import host, upload

pytestmark = pytest.mark.gpu

FP32_GATE = 1e-5


def say(*a):
    print(*a, flush=True)


def forest(n, split):
    """two roots: a chain of `split` nodes, then a random tree below the
    second root (node `split`)"""
    rng = np.random.default_rng(n + split)
    p = gs.random_recursive_tree(rng, n - split, max_depth=20) + split
    p[0] = -1
    return np.concatenate([gs.chain_tree(split), p]).astype(np.int32)


def trees(case):
    rng = np.random.default_rng(321)
    return {
        "n64_mixed": np.stack([gs.chain_tree(64), gs.star_tree(64), gs.kary_bfs_tree(64, 8),
                               forest(64, 20), gs.random_recursive_tree(rng, 64, max_depth=24)]),
        "chain33": np.stack([gs.chain_tree(33)] * 2),
        "n50_forest": np.stack([forest(50, 31), gs.random_recursive_tree(rng, 50)]),
        "chain17": np.stack([gs.chain_tree(17)] * 3),
        "n1": np.stack([gs.chain_tree(1)] * 2),
    }[case]


def run(g, ts):
    d = upload(ts)
    S_before = d["S0"].clone()
    st = torch.full((ts.parent.shape[0],), -7, dtype=torch.int32, device="cuda")
    out = g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"], status=st)
    out2 = g.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"], d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(d["S0"], S_before)          # the committed state is only read
    assert torch.equal(out, out2)                  # deterministic
    return host(out), host(st)


@pytest.mark.parametrize("case", ["n64_mixed", "chain33", "n50_forest", "chain17", "n1"])
def test_verify_fp32_trees(gpu_lib, case):
    say("fp32 verify", case)
    par = trees(case)
    ts = gs.make_set(par, 4, 128, 128, "fp32", seed=900 + par.shape[1])
    out, st = run(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0] * par.shape[0]
    err = oracle.rel_err(out, ref)
    say("rel err", err)
    assert err <= FP32_GATE
    for b in range(par.shape[0]):
        assert oracle.rel_err(out[b], ref[b]) <= FP32_GATE, b


def test_verify_fp32_layer_b16_n64(gpu_lib):
    """the batch-16, 32-head, 64-node layer with fp32 q/k/v, whole tensor"""
    say("fp32 verify b16 n64")
    ts = gs.make_set(gs.make_trees(2, np.random.default_rng(12)), 32, 128, 128, "fp32", seed=12)
    out, st = run(gpu_lib, ts)
    ref, rst = oracle.verify_set(ts)
    assert st.tolist() == rst.tolist() == [0] * 16
    err = oracle.rel_err(out, ref)
    say("rel err", err)
    assert err <= FP32_GATE


def test_verify_fp32_bad_parent(gpu_lib):
    """a malformed tree gets NaN rows and the flag; the others are exact"""
    say("fp32 verify bad parent")
    rng = np.random.default_rng(5)
    par = np.stack([gs.random_recursive_tree(rng, 40) for _ in range(3)])
    par[1, 30] = 30          # a node that is its own parent
    ts = gs.make_set(par, 2, 128, 128, "fp32", seed=5)
    d = upload(ts)
    st = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    out = host(gpu_lib.verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                              d["S0"], status=st))
    ref, rst = oracle.verify_set(ts)
    assert host(st).tolist() == rst.tolist() == [0, gpu_lib.FAULT_BAD_PARENT, 0]
    assert np.isnan(out[1]).all()
    for b in (0, 2):
        assert oracle.rel_err(out[b], ref[b]) <= FP32_GATE, b


# ---------------------------------------------------------------------------
# the all-fp32 commit (fp32-MFMA chunked commit, d_k = d_v = 128)
# ---------------------------------------------------------------------------
def run_commit(g, ts, path, plen):
    d = upload(ts)
    S = d["S0"].clone()
    st = torch.full((ts.parent.shape[0],), -7, dtype=torch.int32, device="cuda")
    g.commit(S, torch.from_numpy(path).cuda(), torch.from_numpy(plen).cuda(), d["k"], d["v"],
             d["alpha"], d["beta"], d["parent"], status=st)
    torch.cuda.synchronize()
    return host(S), host(st)


def test_commit_fp32_chunk_edges_n128(gpu_lib):
    """paths of 1, 31, 32, 33, 64, 97 and 128 nodes along 128-node chains:
    one to four 32-node chunks, full and ragged"""
    say("fp32 commit chunk edges")
    acc = np.array([0, 30, 31, 32, 63, 96, 127], np.int32)
    ts = gs.make_set(np.stack([gs.chain_tree(128)] * 7), 2, 128, 128, "fp32", seed=41,
                     accepted=acc)
    path, plen = ts.paths(max_path=128)
    assert plen.tolist() == [1, 31, 32, 33, 64, 97, 128]
    S, st = run_commit(gpu_lib, ts, path, plen)
    Sref, rst = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert st.tolist() == rst.tolist() == [0] * 7
    err = oracle.rel_err(S, Sref)
    say("rel err", err)
    assert err <= FP32_GATE
    for b in range(7):
        assert oracle.rel_err(S[b], Sref[b]) <= FP32_GATE, b


def test_commit_fp32_layer_and_faults(gpu_lib):
    """the batch-16 / 32-head / 64-node layer's accepted branches (whole
    state), with a bad id, a path that does not start at a root, a broken
    parent link and an empty path: those states bit-unchanged"""
    say("fp32 commit layer + faults")
    ts = gs.make_set(gs.make_trees(2, np.random.default_rng(13)), 32, 128, 128, "fp32", seed=13)
    path, plen = ts.paths(max_path=13)
    path[1, plen[1] - 1] = 64                  # id out of range
    path[2, 0] = path[2, 1] if plen[2] > 1 else 5   # first node not a root
    if plen[3] > 2:
        path[3, 2] = path[3, 1]               # repeated id: the link is broken
    else:
        plen[3] = 14                          # longer than max_path
    plen[4] = 0
    S, st = run_commit(gpu_lib, ts, path, plen)
    Sref, rst = oracle.commit_set(ts, path_arr=path, path_len=plen)
    assert st.tolist() == rst.tolist()
    assert st.tolist()[:5] == [0] + [gpu_lib.FAULT_BAD_PATH] * 3 + [0]
    for b in range(1, 5):
        assert np.array_equal(S[b], ts.S0[b]), b
    err = oracle.rel_err(S, Sref)
    say("rel err", err)
    assert err <= FP32_GATE
