"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, never against the oracle itself or the GPU path.

Citations are to the DFlash-TfM summary page, section "Verifica dell'Albero
Senza Rollback per GDN" (rollback-free tree verification for GDN): the state
update formula, the topological order, the ancestor interaction matrices X
and Y, the system (I+X)U = beta V solved without updating the state, and the
delayed commit along the accepted branch.
"""
import json
import os

import numpy as np
import pytest

import gdn_synth as gs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EXACT = dict(rtol=0, atol=0)


def _rand_set(seed, parent, H=2, dk=6, dv=5):
    return gs.make_set(np.asarray(parent)[None, :] if np.ndim(parent) == 1 else parent,
                       H, dk, dv, "fp32", seed)


# ---------------------------------------------------------------------------
# 1. the hand-worked example (pencil arithmetic, fixture carries the steps)
# ---------------------------------------------------------------------------
def _golden():
    with open(os.path.join(GOLDEN, "hand_tree3_d2.json")) as f:
        g = json.load(f)
    n = len(g["parent"])
    q = np.array(g["q"], float).reshape(1, n, 1, 2)
    k = np.array(g["k"], float).reshape(1, n, 1, 2)
    v = np.array(g["v"], float).reshape(1, n, 1, 2)
    a = np.array(g["alpha"], float).reshape(1, n, 1)
    b = np.array(g["beta"], float).reshape(1, n, 1)
    p = np.array(g["parent"], np.int32).reshape(1, n)
    S0 = np.array(g["S0"], float).reshape(1, 1, 2, 2)
    return g, q, k, v, a, b, p, S0


@pytest.mark.parametrize("memo", [True, False])
def test_golden_hand_example_verify(memo):
    g, q, k, v, a, b, p, S0 = _golden()
    out, st = oracle.verify(q, k, v, a, b, p, S0, memo=memo)
    assert st[0] == 0
    np.testing.assert_allclose(out[0, :, 0, :], np.array(g["out"]), rtol=0, atol=1e-14)
    ob, _ = oracle.brute_verify(q, k, v, a, b, p, S0)
    np.testing.assert_allclose(ob[0, :, 0, :], np.array(g["out"]), rtol=0, atol=1e-14)


def test_golden_hand_example_commit_and_index():
    g, q, k, v, a, b, p, S0 = _golden()
    for key, want in g["commit"].items():
        path = np.array([want["path"]], np.int32)
        S, st = oracle.commit(S0, path, np.array([path.shape[1]], np.int32), k, v, a, b, p)
        assert st[0] == 0
        np.testing.assert_allclose(S[0, 0], np.array(want["S"]), rtol=0, atol=1e-14)
    depth, anc, st = oracle.index(p)
    assert depth[0].tolist() == g["depth"]
    assert anc[0, :, 0].tolist() == g["anc_bits"]


# ---------------------------------------------------------------------------
# 2. brute force: every root-to-leaf branch run separately
# ---------------------------------------------------------------------------
def test_memo_equals_literal_bitwise():
    ts = gs.make_config(1, heads=4)
    o1, _ = oracle.verify_set(ts, memo=True)
    o2, _ = oracle.verify_set(ts, memo=False)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("chain", [False, True])
def test_config0_vs_branch_brute_force(chain):
    ts = gs.make_config(0, chain=chain)
    out, st = oracle.verify_set(ts)
    ob, sb = oracle.brute_verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, ts.S0)
    assert st.tolist() == sb.tolist() == [0]
    assert oracle.rel_err(out, ob) < 1e-13


@pytest.mark.parametrize("seed", range(12))
def test_random_small_trees_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 13))
    parent = gs.random_recursive_tree(rng, n)
    if seed % 3 == 0 and n > 3:                      # a forest: several roots
        parent[n // 2] = -1
    ts = _rand_set(100 + seed, parent, H=3, dk=int(rng.integers(1, 9)), dv=int(rng.integers(1, 9)))
    out, _ = oracle.verify_set(ts)
    ob, _ = oracle.brute_verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, ts.S0)
    assert oracle.rel_err(out, ob) < 1e-13


# ---------------------------------------------------------------------------
# 3. chain tree == ordinary sequential GDN decoding
# ---------------------------------------------------------------------------
def test_chain_equals_sequential_decoding():
    n, H, d = 24, 2, 8
    ts = _rand_set(7, gs.chain_tree(n), H=H, dk=d, dv=d)
    out, _ = oracle.verify_set(ts)
    for h in range(H):
        S = ts.S0[0, h].astype(float)
        for t in range(n):
            kk, vv = ts.k[0, t, h].astype(float), ts.v[0, t, h].astype(float)
            a, b = float(ts.alpha[0, t, h]), float(ts.beta[0, t, h])
            # token-by-token decoding: decay, erase along k, write v along k
            S = a * S - a * b * np.outer(kk, kk @ S) + b * np.outer(kk, vv)
            np.testing.assert_allclose(out[0, t, h], S.T @ ts.q[0, t, h], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# 4. closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_closed_form_query_equals_key_beta_one(seed):
    """q_i = k_i, beta = 1, |k| = 1: S_i^T k_i = alpha (S_p^T (I - k k^T) k) + v = v_i
    for every alpha and S0, on any tree."""
    rng = np.random.default_rng(seed)
    parent = gs.random_recursive_tree(rng, 16)
    ts = _rand_set(seed, parent, H=2, dk=7, dv=5)
    k = ts.k.astype(float)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    out, _ = oracle.verify(k, k, ts.v, ts.alpha, np.ones_like(ts.beta), ts.parent, ts.S0)
    np.testing.assert_allclose(out, ts.v.astype(float), rtol=0, atol=1e-13)


def test_closed_form_single_node():
    """n = 1: o = alpha S0^T q + beta (q.k) (v - alpha S0^T k)."""
    ts = _rand_set(3, np.array([-1]), H=4, dk=9, dv=6)
    out, _ = oracle.verify_set(ts)
    for h in range(4):
        q, k, v = (x[0, 0, h].astype(float) for x in (ts.q, ts.k, ts.v))
        a, b = float(ts.alpha[0, 0, h]), float(ts.beta[0, 0, h])
        S0 = ts.S0[0, h].astype(float)
        want = a * S0.T @ q + b * (q @ k) * (v - a * S0.T @ k)
        np.testing.assert_allclose(out[0, 0, h], want, rtol=1e-13, atol=1e-14)


def test_beta_zero_alpha_one_is_plain_matmul():
    ts = gs.make_config(1, heads=3)
    out, _ = oracle.verify(ts.q, ts.k, ts.v, np.ones_like(ts.alpha), np.zeros_like(ts.beta),
                           ts.parent, ts.S0)
    want = np.einsum("bnhk,bhkv->bnhv", ts.q.astype(float), ts.S0.astype(float))
    assert oracle.rel_err(out, want) < 1e-13


def test_beta_zero_gives_path_decay_times_readout():
    ts = gs.make_config(1, heads=2)
    out, _ = oracle.verify(ts.q, ts.k, ts.v, ts.alpha, np.zeros_like(ts.beta), ts.parent, ts.S0)
    for i in range(ts.parent.shape[1]):
        decay = np.ones(2)
        for t in gs.path_to(ts.parent[0], i):
            decay *= ts.alpha[0, t, :2]
        for h in range(2):
            want = decay[h] * ts.S0[0, h].astype(float).T @ ts.q[0, i, h]
            np.testing.assert_allclose(out[0, i, h], want, rtol=1e-12, atol=1e-14)


def test_orthonormal_keys_write_rows():
    """alpha = 1, beta = 1, S0 = 0 and k_s = e_{depth(s)}: the keys on any path
    are orthonormal, so S_i = sum_{s on path(i)} e_{depth(s)} v_s^T and
    o_i = sum_s q_i[depth(s)] v_s."""
    rng = np.random.default_rng(5)
    parent = gs.random_recursive_tree(rng, 20, max_depth=6)
    ts = _rand_set(5, parent, H=1, dk=8, dv=4)
    depth = gs._depths(parent)
    k = np.zeros_like(ts.k, dtype=float)
    for i in range(20):
        k[0, i, 0, depth[i]] = 1.0
    out, _ = oracle.verify(ts.q, k, ts.v, np.ones_like(ts.alpha), np.ones_like(ts.beta),
                           ts.parent, np.zeros_like(ts.S0))
    for i in range(20):
        want = sum(ts.q[0, i, 0, depth[s]] * ts.v[0, s, 0].astype(float)
                   for s in gs.path_to(parent, i))
        np.testing.assert_allclose(out[0, i, 0], want, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# 5. the chunked form (independent derivation: X, Y, (I+X)U = RHS, output)
# ---------------------------------------------------------------------------
def chunked_form(q, k, v, alpha, beta, parent, S0):
    """Own algebra from the update formula: with u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t)
    the state is S_t = alpha_t S_{t-1} + k_t u_t^T; with g_i the log-decay summed
    over the path of i,
        u_i + beta_i sum_{s in anc(i)} e^{g_i-g_s} (k_i.k_s) u_s = beta_i (v_i - e^{g_i} S0^T k_i)
        o_i = e^{g_i} S0^T q_i + sum_{s in anc*(i)} e^{g_i-g_s} (q_i.k_s) u_s."""
    batch, n, H, dk = q.shape
    out = np.zeros(v.shape, float)
    for b in range(batch):
        paths = [gs.path_to(parent[b], i) for i in range(n)]
        for h in range(H):
            Q, K, V = (x[b, :, h].astype(float) for x in (q, k, v))
            la = np.log(alpha[b, :, h].astype(float))
            g = np.array([la[p].sum() for p in paths])
            bt = beta[b, :, h].astype(float)
            X = np.zeros((n, n))
            Y = np.zeros((n, n))
            for i in range(n):
                for s in paths[i]:
                    w = np.exp(g[i] - g[s])
                    Y[i, s] = w * Q[i] @ K[s]
                    if s != i:
                        X[i, s] = bt[i] * w * K[i] @ K[s]
            S = S0[b, h].astype(float)
            rhs = bt[:, None] * (V - np.exp(g)[:, None] * (K @ S))
            U = np.linalg.solve(np.eye(n) + X, rhs)
            out[b, :, h] = np.exp(g)[:, None] * (Q @ S) + Y @ U
    return out


@pytest.mark.parametrize("cfg", [0, 1])
def test_chunked_form_matches_oracle(cfg):
    ts = gs.make_config(cfg, heads=4)
    out, _ = oracle.verify_set(ts)
    want = chunked_form(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, ts.S0)
    assert oracle.rel_err(out, want) < 1e-11


def test_chunked_form_deep_chain_and_bushes():
    n = 40
    for parent in (gs.chain_tree(n), gs.star_tree(n), gs.kary_bfs_tree(n, 4)):
        ts = _rand_set(11, parent, H=2, dk=8, dv=8)
        out, _ = oracle.verify_set(ts)
        want = chunked_form(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, ts.S0)
        assert oracle.rel_err(out, want) < 1e-11


# ---------------------------------------------------------------------------
# 6. structural invariants
# ---------------------------------------------------------------------------
def _relabel(parent, rng):
    n = len(parent)
    placed, order = set(), []
    ready = [i for i in range(n) if parent[i] < 0]
    while ready:
        j = ready.pop(int(rng.integers(0, len(ready))))
        order.append(j)
        placed.add(j)
        ready += [c for c in range(n) if parent[c] == j]
    perm = np.array(order)            # new id -> old id
    inv = np.empty(n, int)
    inv[perm] = np.arange(n)
    newp = np.array([-1 if parent[o] < 0 else inv[parent[o]] for o in perm], np.int32)
    return perm, newp


def test_relabeling_permutes_outputs():
    rng = np.random.default_rng(9)
    ts = gs.make_config(1, heads=3)
    out, _ = oracle.verify_set(ts)
    perm, newp = _relabel(ts.parent[0], rng)
    assert not np.array_equal(perm, np.arange(len(perm)))
    assert all(newp[i] < i for i in range(len(newp)))
    sl = lambda x: x[:, perm]
    o2, _ = oracle.verify(sl(ts.q), sl(ts.k), sl(ts.v), sl(ts.alpha), sl(ts.beta),
                          newp[None], ts.S0)
    assert np.array_equal(o2, out[:, perm])


def test_non_descendants_unaffected():
    ts = gs.make_config(1, heads=2)
    out, _ = oracle.verify_set(ts)
    par = ts.parent[0]
    j = 5
    desc = {i for i in range(len(par)) if j in set(gs.path_to(par, i))}
    q, k, v = ts.q.copy(), ts.k.copy(), ts.v.copy()
    a, b = ts.alpha.copy(), ts.beta.copy()
    k[0, j] = np.roll(k[0, j], 3, axis=-1)
    v[0, j] *= -2.0
    a[0, j] *= 0.5
    b[0, j] = 1.0 - b[0, j]
    o2, _ = oracle.verify(q, k, v, a, b, ts.parent, ts.S0)
    for i in range(len(par)):
        same = np.array_equal(o2[0, i], out[0, i])
        assert same == (i not in desc), i


def test_linear_in_v_and_state():
    ts = gs.make_config(1, heads=2)
    rng = np.random.default_rng(1)
    V2 = rng.standard_normal(ts.v.shape)
    S2 = rng.standard_normal(ts.S0.shape)
    f = lambda V, S: oracle.verify(ts.q, ts.k, V, ts.alpha, ts.beta, ts.parent, S)[0]
    lhs = f(ts.v + 0.5 * V2, ts.S0 + 0.5 * S2)
    rhs = f(ts.v, ts.S0) + 0.5 * f(V2, S2)
    assert oracle.rel_err(lhs, rhs) < 1e-12


def test_output_depends_only_on_own_path_prefix():
    """Every node of the batch tree equals a chain run along its own path."""
    ts = gs.make_config(1, heads=2)
    out, _ = oracle.verify_set(ts)
    for i in (0, 7, 19, 31):
        p = gs.path_to(ts.parent[0], i)
        sl = lambda x: x[:, p]
        o2, _ = oracle.verify(sl(ts.q), sl(ts.k), sl(ts.v), sl(ts.alpha), sl(ts.beta),
                              gs.chain_tree(len(p))[None], ts.S0)
        assert np.array_equal(o2[0, -1], out[0, i])


# ---------------------------------------------------------------------------
# 7. commit: state along the accepted path, then verify from it
# ---------------------------------------------------------------------------
def _subtree(parent, a):
    """descendants of a (excluding a) re-rooted under the committed state"""
    d = [i for i in range(len(parent)) if i != a and a in set(gs.path_to(parent, i))]
    m = {o: j for j, o in enumerate(d)}
    newp = np.array([-1 if parent[o] == a else m[parent[o]] for o in d], np.int32)
    return np.array(d, int), newp


@pytest.mark.parametrize("cfg", [0, 1])
def test_commit_then_verify_subtree(cfg):
    ts = gs.make_config(cfg) if cfg == 0 else gs.make_config(cfg, heads=3)
    out, _ = oracle.verify_set(ts)
    par = ts.parent[0]
    # pick an interior node with descendants
    a = next(i for i in range(1, len(par)) if (par == i).any())
    path = gs.path_to(par, a)[None]
    S_a, st = oracle.commit(ts.S0, path, np.array([path.shape[1]], np.int32), ts.k, ts.v,
                            ts.alpha, ts.beta, ts.parent)
    assert st[0] == 0
    # committed state reads out node a's verify output
    for h in range(ts.q.shape[2]):
        np.testing.assert_allclose(S_a[0, h].T @ ts.q[0, a, h], out[0, a, h], rtol=1e-13, atol=1e-14)
    d, newp = _subtree(par, a)
    sl = lambda x: x[:, d]
    o2, _ = oracle.verify(sl(ts.q), sl(ts.k), sl(ts.v), sl(ts.alpha), sl(ts.beta),
                          newp[None], S_a)
    assert np.array_equal(o2, out[:, d])


def test_commit_composition():
    ts = gs.make_config(1, heads=3)
    par = ts.parent[0]
    leaf = int(ts.accepted[0])
    full = gs.path_to(par, leaf)
    a = int(full[len(full) // 2])
    p1 = gs.path_to(par, a)
    S1, _ = oracle.commit(ts.S0, p1[None], np.array([len(p1)], np.int32), ts.k, ts.v,
                          ts.alpha, ts.beta, ts.parent)
    d, newp = _subtree(par, a)
    m = {o: j for j, o in enumerate(d)}
    p2 = np.array([m[o] for o in full[len(p1):]], np.int32)
    sl = lambda x: x[:, d]
    S12, _ = oracle.commit(S1, p2[None], np.array([len(p2)], np.int32), sl(ts.k), sl(ts.v),
                           sl(ts.alpha), sl(ts.beta), newp[None])
    Sf, _ = oracle.commit(ts.S0, full[None], np.array([len(full)], np.int32), ts.k, ts.v,
                          ts.alpha, ts.beta, ts.parent)
    assert np.array_equal(S12, Sf)


def test_commit_vs_brute_and_empty_path():
    ts = gs.make_config(1, heads=2)
    path, plen = ts.paths()
    S, st = oracle.commit_set(ts)
    Sb, sb = oracle.brute_commit(ts.S0, path, plen, ts.k, ts.v, ts.alpha, ts.beta, ts.parent)
    assert st[0] == sb[0] == 0
    assert oracle.rel_err(S, Sb) < 1e-13
    S0, st = oracle.commit(ts.S0, path, np.zeros(1, np.int32), ts.k, ts.v, ts.alpha,
                           ts.beta, ts.parent)
    assert st[0] == 0 and np.array_equal(S0, ts.S0.astype(float))


# ---------------------------------------------------------------------------
# 8. faults and tree indexing
# ---------------------------------------------------------------------------
def test_verify_bad_parent_faults_only_that_sequence():
    ts = gs.make_config(2, batch=3, heads=2)
    par = ts.parent.copy()
    par[1, 10] = 12                     # parent after child
    out, st = oracle.verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, par, ts.S0)
    assert st.tolist() == [0, 1, 0]
    assert np.isnan(out[1]).all() and np.isfinite(out[[0, 2]]).all()
    par[2, 0] = -2
    _, st = oracle.verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, par, ts.S0)
    assert st.tolist() == [0, 1, 1]


@pytest.mark.parametrize("case", ["unconnected", "not_root", "id_range", "too_long",
                                  "negative", "not_increasing"])
def test_commit_bad_path_leaves_state(case):
    ts = gs.make_config(2, batch=2, heads=2)
    path, plen = ts.paths(max_path=16)
    p = path.copy()
    L = plen.copy()
    if case == "unconnected":
        p[0, 2] = p[0, 3] if L[0] > 3 else 63
    elif case == "not_root":
        p[0, 0] = p[0, 1]
    elif case == "id_range":
        p[0, 1] = 64
    elif case == "too_long":
        L[0] = 17
    elif case == "negative":
        L[0] = -1
    elif case == "not_increasing":
        par = ts.parent.copy()
        par[0, 1], par[0, 2] = 2, 0      # 0 -> 2 -> 1 (1's parent is later)
        p[0, :3] = [0, 2, 1]
        L[0] = 3
        S, st = oracle.commit(ts.S0, p, L, ts.k, ts.v, ts.alpha, ts.beta, par)
        assert st.tolist() == [2, 0]
        assert np.array_equal(S[0], ts.S0[0].astype(float))
        return
    S, st = oracle.commit(ts.S0, p, L, ts.k, ts.v, ts.alpha, ts.beta, ts.parent)
    Sb, sb = oracle.brute_commit(ts.S0, p, L, ts.k, ts.v, ts.alpha, ts.beta, ts.parent)
    assert st.tolist() == sb.tolist() == [2, 0]
    assert np.array_equal(S[0], ts.S0[0].astype(float))
    assert not np.array_equal(S[1], ts.S0[1].astype(float))


@pytest.mark.parametrize("seed", range(8))
def test_path_and_index_vs_brute(seed):
    rng = np.random.default_rng(seed)
    batch, n = 6, int(rng.integers(1, 70))
    par = np.stack([gs.random_recursive_tree(rng, n) for _ in range(batch)])
    acc = rng.integers(0, n, size=batch).astype(np.int32)
    if n > 4:
        par[1, n - 1] = n - 1            # self parent: malformed
        par[2, 3] = -3
        acc[1] = n - 1
        acc[3] = n                       # out of range
    for mp in (1, 4, n + 1):
        a = oracle.path(par, acc, mp)
        b = oracle.brute_path(par, acc, mp)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    a = oracle.index(par)
    b = oracle.brute_index(par)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_generators_topological_and_deterministic():
    for i in range(5):
        t1 = gs.make_config(i)
        t2 = gs.make_config(i)
        assert np.array_equal(t1.parent, t2.parent)
        assert np.array_equal(t1.q, t2.q) and np.array_equal(t1.S0, t2.S0)
        for par in t1.parent:
            assert par[0] == -1 and all(-1 <= par[j] < j for j in range(len(par)))
    d, _, _ = oracle.index(gs.make_config(2).parent)
    assert d.max() <= 12
    d, _, _ = oracle.index(gs.make_config(1).parent)
    assert d.max() <= 8
    d, _, _ = oracle.index(gs.make_config(3).parent)
    assert d[:16].max() == 127 and d[32:].max() <= 16


# ---------------------------------------------------------------------------
# greedy acceptance walk (integer; pinned by brute force over all paths)
# ---------------------------------------------------------------------------
def _brute_accept(par, draft, verify):
    """every node whose whole path from node 0 matches (each edge p -> c has
    draft[c] == verify[p]); with distinct sibling tokens these nodes form one
    chain, whose deepest node is the accepted one"""
    n = len(par)
    ok = []
    for i in range(n):
        path = gs.path_to(par, i)
        if path[0] != 0:
            continue
        if all(draft[c] == verify[p] for p, c in zip(path[:-1], path[1:])):
            ok.append(i)
    deepest = max(ok, key=lambda i: len(gs.path_to(par, i)))
    return deepest, len(gs.path_to(par, deepest)), int(verify[deepest]), ok


@pytest.mark.parametrize("seed", range(6))
def test_accept_vs_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    par = np.stack([gs.best_first_tree(rng, 40, 4, 10) for _ in range(4)]
                   + [gs.random_recursive_tree(rng, 40) for _ in range(4)])
    draft, verify = gs.make_accept_tokens(rng, par, vocab=50, p_match=0.8)
    acc, alen, bonus, st = oracle.accept(par, draft, verify)
    assert st.tolist() == [0] * 8
    for b in range(8):
        d, L, t, ok = _brute_accept(par[b], draft[b], verify[b])
        # the matching nodes form a single chain from node 0
        depths = sorted(len(gs.path_to(par[b], i)) for i in ok)
        assert depths == list(range(1, len(ok) + 1))
        assert (acc[b], alen[b], bonus[b]) == (d, L, t)


def test_accept_chain_and_star():
    n = 12
    par = gs.chain_tree(n)[None]
    draft = np.arange(100, 100 + n, dtype=np.int32)[None]
    verify = np.full((1, n), 7, np.int32)
    verify[0, :5] = draft[0, 1:6]          # nodes 1..5 match, node 6 does not
    acc, alen, bonus, _ = oracle.accept(par, draft, verify)
    assert (acc[0], alen[0], bonus[0]) == (5, 6, 7)
    star = gs.star_tree(6)[None]
    d2 = np.array([[9, 10, 11, 12, 13, 14]], np.int32)
    v2 = np.array([[13, 0, 0, 0, 0, 0]], np.int32)
    acc, alen, bonus, _ = oracle.accept(star, d2, v2)
    assert (acc[0], alen[0], bonus[0]) == (4, 2, 0)
    # no child matches: only the root is accepted
    acc, alen, bonus, _ = oracle.accept(star, d2, np.full((1, 6), 99, np.int32))
    assert (acc[0], alen[0], bonus[0]) == (0, 1, 99)


def test_accept_ties_forests_and_faults():
    # two siblings carry the matching token: the lower id is taken
    par = np.array([[-1, 0, 0, 1, 2]], np.int32)
    draft = np.array([[0, 5, 5, 6, 6]], np.int32)
    verify = np.array([[5, 6, 6, 0, 0]], np.int32)
    acc, alen, _, _ = oracle.accept(par, draft, verify)
    assert (acc[0], alen[0]) == (3, 3)
    # a second root is never reached, whatever its tokens
    par = np.array([[-1, 0, -1, 2]], np.int32)
    draft = np.array([[1, 2, 3, 4]], np.int32)
    verify = np.array([[3, 9, 4, 9]], np.int32)
    acc, alen, _, st = oracle.accept(par, draft, verify)
    assert (acc[0], alen[0], st[0]) == (0, 1, 0)
    # malformed parents
    par = np.array([[-1, 0, 3, 1], [-1, 0, 1, 2]], np.int32)
    z = np.zeros((2, 4), np.int32)
    acc, alen, bonus, st = oracle.accept(par, z, z)
    assert acc.tolist() == [-1, 3] and alen.tolist() == [0, 4] and st.tolist() == [1, 0]
    assert bonus.tolist() == [-1, 0]


# ---------------------------------------------------------------------------
# width-w best-first tree construction (oracle/tree_build.py)
# ---------------------------------------------------------------------------
def _table_replaying_best_first(seed, n, K):
    """the candidate rows best_first_tree draws, node by node (every node
    proposes when max_depth >= n), as a table"""
    rng = np.random.Generator(np.random.PCG64(seed))
    lp = np.full((n, K), -np.inf)
    for i in range(n):
        c = int(rng.geometric(0.5))
        assert c <= K, "seed draws more children than the table holds"
        lp[i, :c] = np.sort(np.log(rng.dirichlet(np.ones(c))))[::-1]
    return lp


@pytest.mark.parametrize("seed,n,w", [(1, 32, 4), (2, 64, 8), (3, 64, 1), (4, 40, 64)])
def test_tree_build_replays_the_best_first_generator(seed, n, w):
    """an independent implementation (the generator interleaves its random
    draws with its own heap) gives the same tree"""
    lp = _table_replaying_best_first(seed, n, 24)
    ref = gs.best_first_tree(np.random.Generator(np.random.PCG64(seed)), n, w, n)
    par, _, _, nb = oracle.build_tree(lp, np.zeros(lp.shape, np.int32), 0, n, w, n,
                                      dtype=np.float64)
    assert nb == n
    assert np.array_equal(par, ref)


def _strict_best_first(lp, n, max_depth):
    """w = 1 by brute force: every step scans all unused candidates of all
    inserted nodes (no heap)"""
    K = lp.shape[1]
    parent, score, depth, used = [-1], [np.float32(0)], [0], set()
    while len(parent) < n:
        best = None
        for i in range(len(parent)):
            if depth[i] + 1 > max_depth:
                continue
            for j in range(K):
                if (i, j) in used or not np.isfinite(lp[i, j]):
                    continue
                s = np.float32(score[i]) + np.float32(lp[i, j])
                if best is None or s > best[0]:      # ties: first in (i, j) order
                    best = (s, i, j)
        if best is None:
            break
        used.add(best[1:])
        parent.append(best[1])
        score.append(best[0])
        depth.append(depth[best[1]] + 1)
    return np.array(parent, np.int32)


@pytest.mark.parametrize("seed", range(3))
def test_tree_build_width_one_is_strict_best_first(seed):
    lp, tok, root = gs.candidate_table(np.random.default_rng(seed), 1, 30, 6)
    for md in (3, 30):
        par, _, _, nb = oracle.build_tree(lp[0], tok[0], root[0], 30, 1, md)
        ref = _strict_best_first(lp[0], 30, md)
        assert np.array_equal(par[:nb], ref)


@pytest.mark.parametrize("w", [2, 8])
def test_tree_build_rounds_take_the_best_available(w):
    """replay the rounds: each popped group is the w best candidates
    available at that round's start, in order; new nodes wait a round"""
    lp, tok, root = gs.candidate_table(np.random.default_rng(20 + w), 1, 48, 8)
    par, tk, sc, nb = oracle.build_tree(lp[0], tok[0], root[0], 48, w, 6)
    assert nb > 40 and tk[0] == root[0]
    depth = [0]
    for i in range(1, nb):
        depth.append(depth[par[i]] + 1)
        assert par[i] < i and depth[i] <= 6
        j = list(tok[0][par[i]]).index(tk[i])
        assert sc[i] == np.float32(sc[par[i]]) + np.float32(lp[0][par[i], j])
    start, inserted = 1, 1
    while start < nb:
        avail = []
        for i in range(inserted):
            if depth[i] + 1 > 6:
                continue
            for j in range(8):
                if np.isfinite(lp[0][i, j]):
                    avail.append((-(np.float32(sc[i]) + np.float32(lp[0][i, j])), i, j))
        taken = {(par[x], list(tok[0][par[x]]).index(tk[x])) for x in range(1, start)}
        avail = sorted(a for a in avail if a[1:] not in taken)
        grp = list(range(start, start + min(w, len(avail), nb - start)))
        assert [(par[x], list(tok[0][par[x]]).index(tk[x])) for x in grp] == \
            [a[1:] for a in avail[:len(grp)]]
        inserted = start + len(grp)
        start += len(grp)


def _tie_golden():
    """the hand-worked tie cases: tables, tokens and expected arrays (null =
    -inf / absent slot)"""
    with open(os.path.join(GOLDEN, "tree_build_ties.json")) as f:
        g = json.load(f)
    out = []
    for c in g["cases"]:
        lp = np.array([[-np.inf if x is None else x for x in row] for row in c["cand_logp"]],
                      np.float32)
        ii, jj = np.meshgrid(np.arange(lp.shape[0]), np.arange(lp.shape[1]), indexing="ij")
        tok = np.where(np.isfinite(lp), 100 + 10 * ii + jj, -1).astype(np.int32)
        sc = np.array([-np.inf if x is None else x for x in c["score"]], np.float32)
        out.append((c, lp, tok, sc))
    return out


@pytest.mark.parametrize("case", [0, 1, 2])
def test_tree_build_tie_order_hand_worked(case):
    """ties between equal scores go to the lower node id, then the lower slot
    (hand-derived fixture; a reversed tie order changes every case), also
    when two log-probs of one row differ but their fp32 sums with the
    node's score round to the same value (case 2)"""
    c, lp, tok, sc = _tie_golden()[case]
    par, tk, s, nb = oracle.build_tree(lp, tok, c["root_tok"], c["n"], c["width"],
                                       c["max_depth"])
    assert nb == c["n_built"]
    assert par.tolist() == c["parent"]
    assert tk.tolist() == c["token"]
    assert np.array_equal(s, sc)


@pytest.mark.parametrize("seed", range(4))
def test_tree_build_width_one_ties_are_strict_best_first(seed):
    """w = 1 on tables of small integer log-probs (most scores tie): the heap
    matches the brute-force scan, whose ties go to the first (node, slot)"""
    rng = np.random.default_rng(100 + seed)
    lp = rng.choice(np.array([-1, -2, -3, -np.inf], np.float32), size=(24, 4))
    lp[0, 0] = -1                              # the root proposes something
    tok = np.arange(lp.size, dtype=np.int32).reshape(lp.shape)
    for md in (2, 24):
        par, _, _, nb = oracle.build_tree(lp, tok, 0, 24, 1, md)
        ref = _strict_best_first(lp, 24, md)
        assert nb == len(ref)
        assert np.array_equal(par[:nb], ref)


def test_tree_build_runs_dry_and_depth_cap():
    lp = np.full((10, 3), -np.inf, np.float32)
    lp[0, :2] = [-0.1, -0.5]
    lp[1, 0] = -0.2
    par, tk, sc, nb = oracle.build_tree(lp, np.arange(30).reshape(10, 3), 7, 10, 4, 5)
    assert nb == 4 and par.tolist()[:4] == [-1, 0, 0, 1]
    assert par[4:].tolist() == [-1] * 6 and tk[4:].tolist() == [-1] * 6
    assert np.isneginf(sc[4:]).all()
    lp2, tok2, root2 = gs.candidate_table(np.random.default_rng(7), 1, 64, 8)
    par, _, _, nb = oracle.build_tree(lp2[0], tok2[0], root2[0], 64, 8, 1)
    assert (par[1:nb] == 0).all()        # depth cap 1: a star under the root


# ---------------------------------------------------------------------------
# pseudo-values u (what the next iteration's commit can reuse)
# ---------------------------------------------------------------------------
def _decay_path(ts, b, h, path):
    return np.cumsum(np.log(ts.alpha[b, path, h].astype(np.float64)))


@pytest.mark.parametrize("seed", range(3))
def test_pseudo_values_rebuild_the_committed_state(seed):
    """e^{g_a} S0 + sum_{s in path(a)} e^{g_a - g_s} k_s u_s^T equals the
    explicit recurrence along path(a) (the commit oracle), for every node a"""
    rng = np.random.default_rng(70 + seed)
    par = np.stack([gs.random_recursive_tree(rng, 14, max_depth=6) for _ in range(2)])
    ts = gs.make_set(par, 2, 8, 6, "fp32", seed=70 + seed)
    U, st = oracle.pseudo_set(ts)
    assert st.tolist() == [0, 0]
    for b in range(2):
        for a in range(14):
            path = gs.path_to(ts.parent[b], a)
            Sref, _ = oracle.commit(ts.S0[b:b + 1], path[None].astype(np.int32),
                                    np.array([len(path)], np.int32), ts.k[b:b + 1],
                                    ts.v[b:b + 1], ts.alpha[b:b + 1], ts.beta[b:b + 1],
                                    ts.parent[b:b + 1])
            for h in range(2):
                g = _decay_path(ts, b, h, path)
                S = np.exp(g[-1]) * ts.S0[b, h].astype(np.float64)
                for j, s in enumerate(path):
                    S += np.exp(g[-1] - g[j]) * np.outer(ts.k[b, s, h], U[b, s, h])
                np.testing.assert_allclose(S, Sref[0, h], rtol=1e-12, atol=1e-13)


def test_pseudo_values_give_the_outputs():
    """o_i = e^{g_i} S0^T q_i + sum_{s in anc*(i)} e^{g_i - g_s} (q_i . k_s) u_s
    equals the explicit walk's outputs"""
    ts = gs.make_config(0)
    U, _ = oracle.pseudo_set(ts)
    out, _ = oracle.verify_set(ts)
    par = ts.parent[0]
    for i in range(len(par)):
        path = gs.path_to(par, i)
        g = _decay_path(ts, 0, 0, path)
        qi = ts.q[0, i, 0].astype(np.float64)
        o = np.exp(g[-1]) * ts.S0[0, 0].T.astype(np.float64) @ qi
        for j, s in enumerate(path):
            o += np.exp(g[-1] - g[j]) * float(qi @ ts.k[0, s, 0].astype(np.float64)) * U[0, s, 0]
        np.testing.assert_allclose(o, out[0, i, 0], rtol=1e-12, atol=1e-13)


def test_pseudo_values_bad_tree():
    ts = gs.make_config(2, batch=2, heads=2)
    ts.parent[1, 5] = 9
    U, st = oracle.pseudo_set(ts)
    assert st.tolist() == [0, 1] and np.isnan(U[1]).all() and np.isfinite(U[0]).all()
