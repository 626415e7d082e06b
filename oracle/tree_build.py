"""Width-w best-first draft-tree construction, plain heap form.

TEST INFRASTRUCTURE (see the package docstring): the reference the device
tree builder is checked against.

What it computes (DFlash-TfM page, "Costruzione dell'Albero"): the tree is
grown from a candidate heap; instead of expanding one best candidate at a
time, each round takes the top-w candidates off the heap and expands them
together, so a budget of B nodes takes ceil(B / w) sequential rounds.

Reading adopted for the inputs, which the pages leave to the drafter: row i
of the candidate table holds the K child candidates that node i proposes
when it is expanded (log-probabilities, -inf for an absent slot, and token
ids); node ids are insertion order, so row i is read once node i exists.
  * node 0 is the root: score 0, depth 0, its token is root_tok;
  * an inserted node i pushes its candidates j (table order) with score
    score(i) + logp[i][j] and depth depth(i) + 1, unless that depth exceeds
    max_depth;
  * a round pops up to w candidates, best first: higher score, ties by
    earlier push; the popped candidates become nodes in pop order, and only
    after the round do the new nodes push their own candidates;
  * the walk stops at B nodes, or earlier if the heap runs dry (n_built < B;
    the unused rows get parent -1, token -1, score -inf).
Scores are accumulated in the dtype given (float32 to take every ordering
decision exactly as the device does, float64 for the comparison with the
float64 synthetic generator); one addition per node, parent score first.
"""
from __future__ import annotations

import heapq

import numpy as np


def build_tree(cand_logp, cand_tok, root_tok, n, width, max_depth, dtype=np.float32):
    """One sequence.  cand_logp, cand_tok: [n][K].  Returns (parent, token,
    score, n_built)."""
    lp = np.asarray(cand_logp)
    tk = np.asarray(cand_tok)
    K = lp.shape[1]
    parent = [-1]
    token = [int(root_tok)]
    score = [dtype(0.0)]
    depth = [0]
    heap = []
    counter = 0

    def push(node):
        nonlocal counter
        if node >= lp.shape[0] or depth[node] + 1 > max_depth:
            return
        for j in range(K):
            v = lp[node, j]
            if not np.isfinite(v):
                continue
            s = dtype(score[node]) + dtype(v)          # one addition, in dtype
            heapq.heappush(heap, (-float(s), counter, node, j))
            counter += 1

    push(0)
    while len(parent) < n and heap:
        popped = []
        while heap and len(popped) < width and len(parent) + len(popped) < n:
            popped.append(heapq.heappop(heap))
        new_ids = []
        for negs, _, par, j in popped:
            parent.append(par)
            token.append(int(tk[par, j]))
            score.append(dtype(-negs))
            depth.append(depth[par] + 1)
            new_ids.append(len(parent) - 1)
        for node in new_ids:
            push(node)
    n_built = len(parent)
    par_out = np.full(n, -1, np.int32)
    tok_out = np.full(n, -1, np.int32)
    sc_out = np.full(n, -np.inf, dtype)
    par_out[:n_built] = parent
    tok_out[:n_built] = token
    sc_out[:n_built] = score
    return par_out, tok_out, sc_out, n_built


def build_trees(cand_logp, cand_tok, root_tok, width, max_depth, dtype=np.float32):
    """Batched: cand_logp, cand_tok [batch][n][K], root_tok [batch]."""
    lp = np.asarray(cand_logp)
    batch, n, _ = lp.shape
    outs = [build_tree(lp[b], cand_tok[b], root_tok[b], n, width, max_depth, dtype)
            for b in range(batch)]
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]),
            np.stack([o[2] for o in outs]), np.array([o[3] for o in outs], np.int32))
