"""NumPy per-branch brute force (TEST INFRASTRUCTURE, fp64, tiny inputs only).

Written independently of gdn_oracle.c: instead of walking each node's path,
it enumerates every root-to-leaf branch of the tree and runs the GDN update
(DFlash-TfM page, rollback-free GDN verification section, the state-update
formula) along the whole branch, reading each node's output o = S^T q off the
branch as it passes.  A node lying on several branches must get the same
output from each; that is checked here too.
"""
from __future__ import annotations

import numpy as np


def _children(parent):
    ch = [[] for _ in parent]
    for i, p in enumerate(parent):
        if p >= 0:
            ch[int(p)].append(i)
    return ch


def _branches(parent):
    """all root-to-leaf node lists, found by explicit descent from each root"""
    ch = _children(parent)
    out = []
    stack = [[r] for r in range(len(parent)) if parent[r] < 0]
    while stack:
        br = stack.pop()
        kids = ch[br[-1]]
        if not kids:
            out.append(br)
        for c in kids:
            stack.append(br + [c])
    return out


def _valid(parent):
    return all(-1 <= int(p) < i for i, p in enumerate(parent))


def _step(S, k, v, a, b):
    # S <- a (I - b k k^T) S + b k v^T, written with an explicit projector
    d = S.shape[0]
    P = np.eye(d) - b * np.outer(k, k)
    return a * (P @ S) + b * np.outer(k, v)


def brute_verify(q, k, v, alpha, beta, parent, S0):
    q, k, v, alpha, beta, S0 = (np.asarray(x, dtype=np.float64)
                                for x in (q, k, v, alpha, beta, S0))
    parent = np.asarray(parent)
    batch, n, H, dk = q.shape
    dv = v.shape[-1]
    out = np.full((batch, n, H, dv), np.nan)
    status = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        if not _valid(parent[b]):
            status[b] = 1
            continue
        brs = _branches(parent[b])
        for h in range(H):
            seen = np.zeros(n, dtype=bool)
            for br in brs:
                S = S0[b, h].copy()
                for i in br:
                    S = _step(S, k[b, i, h], v[b, i, h], alpha[b, i, h], beta[b, i, h])
                    o = S.T @ q[b, i, h]
                    if seen[i]:
                        assert np.array_equal(o, out[b, i, h]) or np.allclose(
                            o, out[b, i, h], rtol=1e-12, atol=1e-14)
                    else:
                        out[b, i, h] = o
                        seen[i] = True
    return out, status


def brute_commit(S, path, path_len, k, v, alpha, beta, parent):
    S = np.array(S, dtype=np.float64)
    k, v, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (k, v, alpha, beta))
    batch, n, H, dk = k.shape
    status = np.zeros(batch, dtype=np.int32)
    max_path = path.shape[1]
    for b in range(batch):
        m = int(path_len[b])
        p = [int(x) for x in path[b, :max(m, 0)]]
        ok = 0 <= m <= max_path and all(0 <= x < n for x in p)
        if ok:
            ok = all(int(parent[b, x]) == (p[j - 1] if j else -1) for j, x in enumerate(p))
            ok = ok and all(p[j - 1] < p[j] for j in range(1, m))
        if not ok:
            status[b] = 2
            continue
        for h in range(H):
            for i in p:
                S[b, h] = _step(S[b, h], k[b, i, h], v[b, i, h], alpha[b, i, h], beta[b, i, h])
    return S, status


def brute_path(parent, accepted, max_path):
    parent = np.asarray(parent)
    batch, n = parent.shape
    path = np.full((batch, max_path), -1, dtype=np.int32)
    plen = np.zeros(batch, dtype=np.int32)
    status = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        a = int(accepted[b])
        if not 0 <= a < n:
            status[b] = 2
            continue
        walk = [a]
        bad = False
        while True:
            p = int(parent[b, walk[-1]])
            if not -1 <= p < walk[-1]:
                bad = True
                break
            if p == -1:
                break
            walk.append(p)
        if bad:
            status[b] = 1
            continue
        if len(walk) > max_path:
            status[b] = 2
            continue
        walk.reverse()
        path[b, :len(walk)] = walk
        plen[b] = len(walk)
    return path, plen, status


def brute_index(parent):
    parent = np.asarray(parent)
    batch, n = parent.shape
    W = (n + 31) // 32
    depth = np.full((batch, n), -1, dtype=np.int32)
    anc = np.zeros((batch, n, W), dtype=np.uint32)
    status = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        if not _valid(parent[b]):
            status[b] = 1
            continue
        for i in range(n):
            chain = [i]
            while parent[b, chain[-1]] >= 0:
                chain.append(int(parent[b, chain[-1]]))
            depth[b, i] = len(chain) - 1
            for s in chain:
                anc[b, i, s // 32] |= np.uint32(1 << (s % 32))
    return depth, anc, status
