"""fp64 CPU oracle for Gated DeltaNet tree verify / commit.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import this package.  The product library never
loads it, and this package never imports the product package.

Two independent implementations live here:
  * gdn_oracle.c (loaded through ctypes): the explicit sequential recurrence
    along each node's root-to-node path, fp64, literal or memoised walk.
  * brute.py: a NumPy per-branch brute force (every root-to-leaf branch run
    on its own, each node read off the branch that contains it).
  * tree_build.py: the width-w best-first draft-tree construction as a
    plain heap.

Inputs are widened exactly to fp64 (bf16 -> fp32 -> fp64 loses nothing).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .brute import brute_verify, brute_commit, brute_path, brute_index  # noqa: F401
from .tree_build import build_tree, build_trees  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

BAD_PARENT = 1
BAD_PATH = 2


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c with gcc (fp contraction off, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int
            lib.oracle_verify.argtypes = [P] * 8 + [I] * 7 + [P]
            lib.oracle_verify.restype = I
            lib.oracle_commit.argtypes = [P, P, P, I, P, P, P, P, P] + [I] * 6 + [P]
            lib.oracle_commit.restype = I
            lib.oracle_path.argtypes = [P, P, P, P, I, I, I, P]
            lib.oracle_path.restype = None
            lib.oracle_index.argtypes = [P, P, P, I, I, P]
            lib.oracle_index.restype = None
            lib.oracle_accept.argtypes = [P] * 6 + [I, I, P]
            lib.oracle_accept.restype = None
            lib.oracle_pseudo.argtypes = [P] * 7 + [I] * 6 + [P]
            lib.oracle_pseudo.restype = I
            _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def verify(q, k, v, alpha, beta, parent, S0, memo=True, nthreads=0,
           return_threads=False):
    """Returns (out fp64 [batch][n][H][dv], status int32 [batch])."""
    lib = _load()
    q, k, v, alpha, beta, S0 = map(_f64, (q, k, v, alpha, beta, S0))
    parent = _i32(parent)
    batch, n, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == q.shape[:3]
    assert alpha.shape == (batch, n, H) and beta.shape == (batch, n, H)
    assert parent.shape == (batch, n) and S0.shape == (batch, H, dk, dv)
    out = np.zeros((batch, n, H, dv), dtype=np.float64)
    status = np.zeros(batch, dtype=np.int32)
    used = lib.oracle_verify(_p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(parent),
                             _p(S0), _p(out), batch, n, H, dk, dv, int(bool(memo)),
                             int(nthreads), _p(status))
    if return_threads:
        return out, status, used
    return out, status


def commit(S, path, path_len, k, v, alpha, beta, parent, nthreads=0,
           return_threads=False):
    """Returns (S_new fp64 [batch][H][dk][dv], status).  Input S is not modified."""
    lib = _load()
    S = _f64(S).copy()
    k, v, alpha, beta = map(_f64, (k, v, alpha, beta))
    path, path_len, parent = map(_i32, (path, path_len, parent))
    batch, n, H, dk = k.shape
    dv = v.shape[-1]
    max_path = path.shape[1]
    assert S.shape == (batch, H, dk, dv) and path_len.shape == (batch,)
    status = np.zeros(batch, dtype=np.int32)
    used = lib.oracle_commit(_p(S), _p(path), _p(path_len), max_path, _p(k), _p(v),
                             _p(alpha), _p(beta), _p(parent), batch, n, H, dk, dv,
                             int(nthreads), _p(status))
    if return_threads:
        return S, status, used
    return S, status


def path(parent, accepted, max_path):
    """Returns (path int32 [batch][max_path], path_len int32 [batch], status)."""
    lib = _load()
    parent, accepted = _i32(parent), _i32(accepted)
    batch, n = parent.shape
    out = np.zeros((batch, max_path), dtype=np.int32)
    plen = np.zeros(batch, dtype=np.int32)
    status = np.zeros(batch, dtype=np.int32)
    lib.oracle_path(_p(parent), _p(accepted), _p(out), _p(plen), batch, n, max_path,
                    _p(status))
    return out, plen, status


def index(parent):
    """Returns (depth int32 [batch][n], anc uint32 [batch][n][ceil(n/32)], status)."""
    lib = _load()
    parent = _i32(parent)
    batch, n = parent.shape
    W = (n + 31) // 32
    depth = np.zeros((batch, n), dtype=np.int32)
    anc = np.zeros((batch, n, W), dtype=np.uint32)
    status = np.zeros(batch, dtype=np.int32)
    lib.oracle_index(_p(parent), _p(depth), _p(anc), batch, n, _p(status))
    return depth, anc, status


def pseudo(k, v, alpha, beta, parent, S0, nthreads=0):
    """Pseudo-values u_i = beta_i (v_i - alpha_i S_parent^T k_i) of every node.
    Returns (U fp64 [batch][n][H][dv], status)."""
    lib = _load()
    k, v, alpha, beta, S0 = map(_f64, (k, v, alpha, beta, S0))
    parent = _i32(parent)
    batch, n, H, dk = k.shape
    dv = v.shape[-1]
    U = np.zeros((batch, n, H, dv), dtype=np.float64)
    status = np.zeros(batch, dtype=np.int32)
    lib.oracle_pseudo(_p(k), _p(v), _p(alpha), _p(beta), _p(parent), _p(S0), _p(U), batch, n,
                      H, dk, dv, int(nthreads), _p(status))
    return U, status


def pseudo_set(ts, S0=None, **kw):
    return pseudo(ts.k, ts.v, ts.alpha, ts.beta, ts.parent, ts.S0 if S0 is None else S0, **kw)


def accept(parent, draft, verify):
    """Greedy acceptance walk.  Returns (accepted, accept_len, bonus, status),
    int32 [batch] each."""
    lib = _load()
    parent, draft, verify = _i32(parent), _i32(draft), _i32(verify)
    batch, n = parent.shape
    assert draft.shape == (batch, n) and verify.shape == (batch, n)
    acc = np.zeros(batch, dtype=np.int32)
    alen = np.zeros(batch, dtype=np.int32)
    bonus = np.zeros(batch, dtype=np.int32)
    status = np.zeros(batch, dtype=np.int32)
    lib.oracle_accept(_p(parent), _p(draft), _p(verify), _p(acc), _p(alen), _p(bonus), batch, n,
                      _p(status))
    return acc, alen, bonus, status


def verify_set(ts, **kw):
    """verify() on a gdn_synth.TensorSet"""
    return verify(ts.q, ts.k, ts.v, ts.alpha, ts.beta, ts.parent, ts.S0, **kw)


def commit_set(ts, S=None, path_arr=None, path_len=None, **kw):
    if path_arr is None:
        path_arr, path_len = ts.paths()
    return commit(ts.S0 if S is None else S, path_arr, path_len, ts.k, ts.v,
                  ts.alpha, ts.beta, ts.parent, **kw)


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| over the whole tensor (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    return float(num / den) if den > 0 else float(num)
