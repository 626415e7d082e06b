"""GPU parity of the all-fp32 verify fast path (fp32 q/k/v, d_k = d_v = 128,
n <= 64: the fp32-MFMA kernel) against the fp64 oracle, at the fp32 gate
max|gpu - ref| / max|ref| <= 1e-5 over whole output tensors.

The method is the DFlash-TfM page's rollback-free tree verification for
GDN: the tree is topologically sorted, X and Y follow the ancestor
relations, (I + X) U = beta V (with the committed-state term) is solved
without touching the state.  Shapes: 64-node chains (the last
pointer-jumping rounds and a dense coupling block between the two 32-row
halves), a star, an 8-ary bush, a two-root forest, short chains that leave
the second block empty or ragged, the batch-16 / 32-head / 64-node layer,
malformed parents, and the fused call's fp32 fallback (commit launch, then
this verify ORing its flag into the commit's).
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
