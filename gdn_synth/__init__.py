"""Seeded synthetic inputs for Gated DeltaNet tree verification.

This module only draws numbers: draft trees (parent arrays), q/k/v, the decay
and write-strength gates, the committed state S0 and an accepted leaf.  It
holds none of the verify or commit arithmetic, so both the fp64 oracle and the
GPU path can consume it without sharing any of the method's code.

The workloads stand in for the pages' own evaluation (a 27B GDN verifier on
chat/math/code prompts, tree size up to 126 tokens), which needs weights and
datasets that are not used here: every tensor is drawn from the distributions
below, with the shapes of one GDN layer.

Layouts (all C-contiguous):
  q, k   [batch][n][H][d_k]   bf16 (stored as uint16 bit patterns) or fp32
  v      [batch][n][H][d_v]
  alpha  [batch][n][H]        fp32 in (0, 1)
  beta   [batch][n][H]        fp32 in (0, 1)
  parent [batch][n]           int32, -1 = child of the committed state,
                              topological: parent[i] < i
  S0     [batch][H][d_k][d_v] fp32

Draw order for one tensor set: tree -> q -> k -> v -> z_alpha -> z_beta -> S0
-> accepted leaf, from numpy.random.Generator(PCG64(seed)).

Distributions: q, k ~ N(0, 1) then L2-normalised per (node, head) along d_k in
fp64; v ~ N(0, 1); alpha = exp(-softplus(z)) = sigmoid(-z), beta = sigmoid(z'),
z, z' ~ N(0, 1); S0 ~ N(0, 1/d_k).  Every value is rounded fp64 -> fp32 (round
to nearest even) and, for bf16 tensors, fp32 -> bf16 (round to nearest even),
so that the oracle and the GPU read identical bits.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "TensorSet", "WORKLOADS", "make_set", "make_config",
    "random_recursive_tree", "chain_tree", "star_tree", "kary_bfs_tree",
    "best_first_tree", "mixed_tree_batch", "pick_leaf", "leaves",
    "to_bf16_bits", "bf16_bits_to_f32", "path_to", "select", "slice_set",
]


# ----------------------------------------------------------------------------
# bf16 rounding (round to nearest even on the fp32 bit pattern)
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# tree shapes
# ----------------------------------------------------------------------------
def chain_tree(n: int) -> np.ndarray:
    p = np.arange(-1, n - 1, dtype=np.int32)
    return p


def star_tree(n: int) -> np.ndarray:
    p = np.zeros(n, dtype=np.int32)
    p[0] = -1
    return p


def kary_bfs_tree(n: int, k: int) -> np.ndarray:
    p = np.array([-1] + [(i - 1) // k for i in range(1, n)], dtype=np.int32)
    return p


def _depths(parent: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parent), dtype=np.int64)
    for i, p in enumerate(parent):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


def random_recursive_tree(rng: np.random.Generator, n: int,
                          max_depth: int | None = None) -> np.ndarray:
    """node 0 is the root; node i picks its parent uniformly among earlier
    nodes (restricted to nodes of depth < max_depth when given)."""
    p = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        if max_depth is None:
            j = int(rng.integers(0, i))
        else:
            cand = np.nonzero(depth[:i] < max_depth)[0]
            j = int(cand[rng.integers(0, len(cand))])
        p[i] = j
        depth[i] = depth[j] + 1
    return p


def best_first_tree(rng: np.random.Generator, n: int, width: int,
                    max_depth: int) -> np.ndarray:
    """Draft tree grown by width-w best-first expansion.

    The tree-construction passage of the DFlash-TfM page pops the top-w
    candidates from a candidate heap and expands all w at once, so a budget
    of B nodes takes ceil(B/w) sequential rounds.  Candidate scores here are
    synthetic (no drafter): node 0 is the root with score 0; every inserted
    node proposes c ~ Geometric(1/2) children whose scores are its own score
    plus the log of a Dirichlet(1) split of probability mass over the c
    children, sorted descending.  Candidates deeper than max_depth are not
    proposed.  Each round pops the best w candidates (ties: lower insertion
    counter first) and appends them as new nodes in pop order, so node ids
    are topological.  If the heap runs dry, every node shallower than
    max_depth proposes one extra child with score own + log(U(0,1)).
    """
    parent = [-1]
    score = [0.0]
    depth = [0]
    heap: list[tuple[float, int, int]] = []   # (-score, counter, parent)
    counter = 0

    def propose(node: int) -> None:
        nonlocal counter
        if depth[node] + 1 > max_depth:
            return
        c = int(rng.geometric(0.5))
        split = np.sort(np.log(rng.dirichlet(np.ones(c))))[::-1]
        for s in split:
            heapq.heappush(heap, (-(score[node] + float(s)), counter, node))
            counter += 1

    propose(0)
    while len(parent) < n:
        if not heap:
            for node in range(len(parent)):
                if depth[node] < max_depth:
                    s = score[node] + math.log(float(rng.uniform(1e-12, 1.0)))
                    heapq.heappush(heap, (-s, counter, node))
                    counter += 1
            if not heap:
                raise ValueError("max_depth too small for n nodes")
        batch = []
        while heap and len(batch) < width and len(parent) + len(batch) < n:
            batch.append(heapq.heappop(heap))
        new_ids = []
        for negs, _, par in batch:
            parent.append(par)
            score.append(-negs)
            depth.append(depth[par] + 1)
            new_ids.append(len(parent) - 1)
        for node in new_ids:
            propose(node)
    return np.asarray(parent, dtype=np.int32)


def leaves(parent: np.ndarray) -> np.ndarray:
    has_child = np.zeros(len(parent), dtype=bool)
    for p in parent:
        if p >= 0:
            has_child[p] = True
    return np.nonzero(~has_child)[0].astype(np.int32)


def pick_leaf(rng: np.random.Generator, parent: np.ndarray) -> int:
    """an accepted node chosen uniformly among the tree's leaves"""
    lv = leaves(parent)
    return int(lv[rng.integers(0, len(lv))])


def path_to(parent: np.ndarray, node: int) -> np.ndarray:
    """root -> node list (host helper for building inputs)"""
    out = []
    while node >= 0:
        out.append(node)
        node = int(parent[node])
    return np.asarray(out[::-1], dtype=np.int32)


def mixed_tree_batch(rng: np.random.Generator, batch: int, n: int) -> np.ndarray:
    """A quarter pure chains, a quarter bushes (stars, then 16-ary BFS trees),
    half random recursive trees of depth <= 16."""
    q = batch // 4
    out = np.empty((batch, n), dtype=np.int32)
    for b in range(batch):
        if b < q:
            out[b] = chain_tree(n)
        elif b < q + q // 2:
            out[b] = star_tree(n)
        elif b < 2 * q:
            out[b] = kary_bfs_tree(n, 16)
        else:
            out[b] = random_recursive_tree(rng, n, max_depth=16)
    return out


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------
@dataclass
class TensorSet:
    """One seeded input set.  *_bits hold bf16 patterns (uint16) when
    dtype == 'bf16'; q/k/v always hold the exact fp32 values."""
    dtype: str
    parent: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    S0: np.ndarray
    accepted: np.ndarray
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        b, n, h, dk = self.q.shape
        return b, n, h, dk, self.v.shape[-1]

    def paths(self, max_path: int | None = None):
        """(path [batch][max_path] int32 padded with -1, path_len [batch])"""
        b = self.parent.shape[0]
        ps = [path_to(self.parent[i], int(self.accepted[i])) for i in range(b)]
        m = max(len(p) for p in ps) if max_path is None else max_path
        path = np.full((b, m), -1, dtype=np.int32)
        plen = np.zeros(b, dtype=np.int32)
        for i, p in enumerate(ps):
            path[i, :len(p)] = p
            plen[i] = len(p)
        return path, plen


def _round_tensor(x64: np.ndarray, dtype: str):
    x32 = x64.astype(np.float32)
    if dtype == "fp32":
        return x32, None
    bits = to_bf16_bits(x32)
    return bf16_bits_to_f32(bits).reshape(x32.shape), bits.reshape(x32.shape)


def make_set(parent: np.ndarray, H: int, d_k: int, d_v: int, dtype: str,
             seed: int, rng: np.random.Generator | None = None,
             accepted: np.ndarray | None = None) -> TensorSet:
    """Draw q, k, v, alpha, beta, S0 and an accepted leaf for given trees.

    `parent` is [batch][n].  If `rng` is given it continues that stream (the
    tree was drawn from it first); otherwise a fresh PCG64(seed) is used.
    """
    if dtype not in ("fp32", "bf16"):
        raise ValueError(dtype)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    if parent.ndim == 1:
        parent = parent[None, :]
    batch, n = parent.shape
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((batch, n, H, d_k))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((batch, n, H, d_k))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((batch, n, H, d_v))
    za = rng.standard_normal((batch, n, H))
    zb = rng.standard_normal((batch, n, H))
    alpha = (1.0 / (1.0 + np.exp(za))).astype(np.float32)   # sigmoid(-z)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)   # sigmoid(z')
    S0 = (rng.standard_normal((batch, H, d_k, d_v)) / math.sqrt(d_k)).astype(np.float32)
    if accepted is None:
        accepted = np.array([pick_leaf(rng, parent[b]) for b in range(batch)],
                            dtype=np.int32)
    q32, qb = _round_tensor(q, dtype)
    k32, kb = _round_tensor(k, dtype)
    v32, vb = _round_tensor(v, dtype)
    return TensorSet(dtype=dtype, parent=parent, q=q32, k=k32, v=v32,
                     alpha=alpha, beta=beta, S0=S0,
                     accepted=np.asarray(accepted, dtype=np.int32),
                     q_bits=qb, k_bits=kb, v_bits=vb,
                     meta={"seed": seed, "H": H, "d_k": d_k, "d_v": d_v})


# ----------------------------------------------------------------------------
# the five workload shapes
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n: int
    H: int
    d_k: int
    d_v: int
    dtype: str
    layers: int = 1
    description: str = ""


WORKLOADS = [
    Workload("tiny-fp32-b1-h1-d16-n8", 1, 8, 1, 16, 16, "fp32",
             description="8-node random recursive tree (plus the 8-node chain), fp32"),
    Workload("gdn-layer-b1-h32-d128-n32", 1, 32, 32, 128, 128, "bf16",
             description="width-4 best-first tree, max depth 8"),
    Workload("gdn-layer-b16-h32-d128-n64", 16, 64, 32, 128, 128, "bf16",
             description="width-8 best-first trees, max depth 12, per sequence"),
    Workload("gdn-layer-b64-h32-d128-n128", 64, 128, 32, 128, 128, "bf16",
             description="chains / bushes / random recursive trees of depth <= 16"),
    Workload("gdn-stack48-b32-h32-d128-n64", 32, 64, 32, 128, 128, "bf16", layers=48,
             description="48 GDN layers sharing one width-8 best-first tree per sequence"),
]


def make_trees(i: int, rng: np.random.Generator) -> np.ndarray:
    w = WORKLOADS[i]
    if i == 0:
        return random_recursive_tree(rng, w.n)[None, :]
    if i == 1:
        return best_first_tree(rng, w.n, 4, 8)[None, :]
    if i in (2, 4):
        return np.stack([best_first_tree(rng, w.n, 8, 12) for _ in range(w.batch)])
    if i == 3:
        return mixed_tree_batch(rng, w.batch, w.n)
    raise IndexError(i)


def make_config(i: int, s: int = 0, layer: int = 0, chain: bool = False,
                batch: int | None = None, heads: int | None = None) -> TensorSet:
    """Input set for workload i with seed 1000*i + s (+ layer for the stack).

    For the 48-layer stack the trees and accepted leaves come from seed
    1000*i + s and each layer's tensors from seed 1000*i + s + 1 + layer.
    `chain` replaces workload 0's tree by the 8-node chain.  `batch`/`heads`
    take a leading slice of the drawn set (used for bounded samples).
    """
    w = WORKLOADS[i]
    seed = 1000 * i + s
    rng = np.random.Generator(np.random.PCG64(seed))
    parent = make_trees(i, rng)
    if chain:
        parent = chain_tree(w.n)[None, :]
    if i == 4:
        accepted = np.array([pick_leaf(rng, parent[b]) for b in range(w.batch)],
                            dtype=np.int32)
        ts = make_set(parent, w.H, w.d_k, w.d_v, w.dtype, seed + 1 + layer,
                      accepted=accepted)
    else:
        ts = make_set(parent, w.H, w.d_k, w.d_v, w.dtype, seed, rng=rng)
    ts.meta.update({"config": i, "workload": w.name, "layer": layer})
    if batch is not None or heads is not None:
        ts = slice_set(ts, batch, heads)
    return ts


# ----------------------------------------------------------------------------
# token ids for the acceptance walk (synthetic: no model produces them here)
# ----------------------------------------------------------------------------
def make_accept_tokens(rng: np.random.Generator, parent: np.ndarray, vocab: int = 32768,
                       p_match: float = 0.7):
    """Draft token ids per node (siblings distinct) and verifier greedy ids.

    For a node with children the verifier's id equals one child's draft id
    (uniform among the children) with probability p_match, else an id no
    child carries; for a leaf it is uniform.  Returns (draft, verify), int32
    arrays shaped like `parent`.
    """
    parent = np.asarray(parent)
    draft = np.zeros(parent.shape, dtype=np.int32)
    verify = np.zeros(parent.shape, dtype=np.int32)
    for b in range(parent.shape[0]):
        par = parent[b]
        n = len(par)
        kids = [[] for _ in range(n)]
        roots = []
        for i in range(n):
            (kids[par[i]] if par[i] >= 0 else roots).append(i)
        for group in [roots] + kids:
            if group:
                draft[b, group] = rng.choice(vocab, size=len(group), replace=False)
        for i in range(n):
            if kids[i] and rng.random() < p_match:
                verify[b, i] = draft[b, kids[i][int(rng.integers(0, len(kids[i])))]]
            else:
                taken = set(int(x) for x in draft[b, kids[i]])
                t = int(rng.integers(0, vocab))
                while t in taken:
                    t = int(rng.integers(0, vocab))
                verify[b, i] = t
    return draft, verify


def candidate_table(rng: np.random.Generator, batch: int, n: int, K: int,
                    vocab: int = 32768):
    """Synthetic child-candidate table for the tree builder: for every node
    row, c ~ Geometric(1/2) candidates (at most K) whose log-probabilities
    are the log of a Dirichlet(1) split sorted descending, -inf in the other
    slots, and distinct token ids.  Rows are drawn in node order, so with a
    large enough max_depth the table replays best_first_tree's draws.
    Returns (logp float32 [batch][n][K], tok int32 [batch][n][K],
    root_tok int32 [batch])."""
    lp = np.full((batch, n, K), -np.inf, dtype=np.float64)
    tok = np.full((batch, n, K), -1, dtype=np.int32)
    for b in range(batch):
        for i in range(n):
            c = min(int(rng.geometric(0.5)), K)
            lp[b, i, :c] = np.sort(np.log(rng.dirichlet(np.ones(c))))[::-1]
            tok[b, i, :c] = rng.choice(vocab, size=c, replace=False)
    root = rng.integers(0, vocab, size=batch).astype(np.int32)
    return lp.astype(np.float32), tok, root


# Tree-size-126 workload for the tree-vs-branch comparison (the pages time
# their fused kernel against single-branch recurrent verification at 126 tree
# tokens): one layer, batch 16, 32 heads, d 128, bf16, width-8 best-first
# trees of 126 nodes (16 expansion rounds, max depth 16).
TREE126 = Workload("gdn-layer-b16-h32-d128-n126", 16, 126, 32, 128, 128, "bf16",
                   description="width-8 best-first trees of 126 nodes, max depth 16")


def make_tree126(s: int = 0, batch: int | None = None) -> TensorSet:
    """Input set of the 126-node comparison workload, seed 9000 + s."""
    w = TREE126
    b = w.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(9000 + s))
    parent = np.stack([best_first_tree(rng, w.n, 8, 16) for _ in range(b)])
    ts = make_set(parent, w.H, w.d_k, w.d_v, w.dtype, 9000 + s, rng=rng)
    ts.meta.update({"workload": w.name})
    return ts


def slice_set(ts: TensorSet, batch: int | None, heads: int | None) -> TensorSet:
    b = slice(None) if batch is None else slice(0, batch)
    h = slice(None) if heads is None else slice(0, heads)

    def c(x, hdim):
        if x is None:
            return None
        idx = [b] + [slice(None)] * (x.ndim - 1)
        if hdim is not None:
            idx[hdim] = h
        return np.ascontiguousarray(x[tuple(idx)])

    return TensorSet(dtype=ts.dtype, parent=c(ts.parent, None), q=c(ts.q, 2),
                     k=c(ts.k, 2), v=c(ts.v, 2), alpha=c(ts.alpha, 2),
                     beta=c(ts.beta, 2), S0=c(ts.S0, 1),
                     accepted=np.ascontiguousarray(ts.accepted[b]),
                     q_bits=c(ts.q_bits, 2), k_bits=c(ts.k_bits, 2),
                     v_bits=c(ts.v_bits, 2), meta=dict(ts.meta))


def select(ts: TensorSet, seqs) -> TensorSet:
    """the batch elements `seqs` of a set (sequences are independent)"""
    seqs = np.asarray(seqs)
    f = lambda x: None if x is None else np.ascontiguousarray(x[seqs])
    return TensorSet(dtype=ts.dtype, parent=f(ts.parent), q=f(ts.q), k=f(ts.k), v=f(ts.v),
                     alpha=f(ts.alpha), beta=f(ts.beta), S0=f(ts.S0), accepted=f(ts.accepted),
                     q_bits=f(ts.q_bits), k_bits=f(ts.k_bits), v_bits=f(ts.v_bits),
                     meta=dict(ts.meta))
