"""Rollback-free tree verification and commit for Gated DeltaNet on MI355X.

Thin Python binding over the C ABI of libgdntree.so (include/gdn_tree.h).
Every function here only marshals arguments: it checks torch tensors, takes
their device pointers and the current HIP stream, and calls the entry point
of the same name.  All computation runs in the library's HIP kernels; there
is no CPU or PyTorch fallback, and a missing library raises.

    verify(q, k, v, alpha, beta, parent, S0)        -> out   (gdn_tree_verify)
    branch_verify(q, k, v, alpha, beta, parent, S0) -> out   (gdn_branch_verify, baseline)
    commit(S, path, path_len, k, v, alpha, beta, parent)     (gdn_tree_commit, in place)
    commit_verify(S, path, path_len, prev, q, k, v, alpha, beta, parent)
                                                    -> out   (gdn_tree_commit_verify)
    build_tree(cand_logp, cand_tok, root_tok, width, max_depth)
                                                    -> (parent, token, score, n_built)
    accept(parent, draft_tok, verify_tok)           -> (accepted, accept_len, bonus_tok)
    path(parent, accepted, max_path)                -> (path, path_len)
    index(parent)                                   -> (depth, anc)
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["load", "lib_path", "verify", "branch_verify", "commit", "commit_verify", "build_tree", "accept", "path", "Launch", "index", "status_string",
           "GdnError", "FAULT_BAD_PARENT", "FAULT_BAD_PATH", "DTYPE_F32", "DTYPE_BF16",
           "MAX_NODES", "MAX_DIM", "ABI_VERSION", "build"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgdntree.so"

FAULT_BAD_PARENT = 1
FAULT_BAD_PATH = 2
DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2     # pseudo-values of commit_verify only
MAX_NODES = 128
MAX_DIM = 128
MAX_CANDIDATES = 32
# GDN_TREE_ABI_VERSION of include/gdn_tree.h that the signatures below follow
ABI_VERSION = 8

_lock = threading.Lock()
_lib = None


class GdnError(RuntimeError):
    """A negative gdn_status returned by the library."""

    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn}: {text} (status {code})")
        self.code = code


def lib_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def build(verbose: bool = False) -> str:
    """Compile libgdntree.so in-tree (hipcc, gfx950)."""
    from . import _build as _b
    return _b.build(verbose=verbose)


def load() -> ctypes.CDLL:
    """Load libgdntree.so from the package directory (raises if absent)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built; run gated_deltanet_tree_verify_amd.build()")
        lib = ctypes.CDLL(p)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.gdn_tree_verify.argtypes = [P, P, P, I, P, P, P, P, P, I, I, I, I, I, P, P]
        lib.gdn_tree_verify.restype = I
        lib.gdn_branch_verify.argtypes = [P, P, P, I, P, P, P, P, P, I, I, I, I, I, P, P]
        lib.gdn_branch_verify.restype = I
        lib.gdn_tree_commit.argtypes = [P, P, P, I, P, P, I, P, P, P, I, I, I, I, I, P, P]
        lib.gdn_tree_commit.restype = I
        lib.gdn_tree_commit_verify.argtypes = [P, P, P, I, P, P, P, P, P, P, I, P, P, P, I, P, P,
                                               P, P, P, I, I, I, I, I, I, P, P]
        lib.gdn_tree_commit_verify.restype = I
        lib.gdn_tree_build.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
        lib.gdn_tree_build.restype = I
        lib.gdn_tree_accept.argtypes = [P, P, P, P, P, P, I, I, P, P]
        lib.gdn_tree_accept.restype = I
        lib.gdn_tree_path.argtypes = [P, P, P, P, I, I, I, P, P]
        lib.gdn_tree_path.restype = I
        lib.gdn_tree_index.argtypes = [P, P, P, I, I, P, P]
        lib.gdn_tree_index.restype = I
        lib.gdn_status_string.argtypes = [I]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_tree_abi_version.argtypes = []
        lib.gdn_tree_abi_version.restype = I
        got = lib.gdn_tree_abi_version()
        if got != ABI_VERSION:
            raise RuntimeError(f"{p} has ABI version {got}, this binding expects {ABI_VERSION}; "
                               "rebuild with gated_deltanet_tree_verify_amd.build()")
        _lib = lib
        return lib


def status_string(code: int) -> str:
    return load().gdn_status_string(int(code)).decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, code):
    if code != 0:
        raise GdnError(fn, code, status_string(code))


class Launch:
    """One entry-point call with its arguments already checked and marshalled
    (device pointers, sizes, stream).  Calling it re-issues the same launch
    with no per-call checks, for launch loops where those checks would cost
    more host time than the kernel takes on the GPU.  It keeps references to
    its tensors; `result` is what the eager call returns."""

    __slots__ = ("_fn", "_name", "_args", "_keep", "result")

    def __init__(self, name, fn, args, keep, result):
        self._name, self._fn, self._args, self._keep, self.result = name, fn, args, keep, result

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _check(self._name, rc)
        return self.result


def _issue(name, fn, args, keep, result, prepare):
    if prepare:
        return Launch(name, fn, args, keep, result)
    _check(name, fn(*args))
    return result


def _need(t, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _qkv_dtype(q):
    torch = _torch()
    return DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F32


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def _verify_like(name, q, k, v, alpha, beta, parent, S0, out, status, stream, prepare):
    torch = _torch()
    lib = load()
    qk = (torch.bfloat16, torch.float32)
    _need(q, "q", qk)
    batch, n, H, dk = q.shape
    _need(k, "k", (q.dtype,), q.shape)
    _need(v, "v", (q.dtype,))
    if tuple(v.shape[:3]) != (batch, n, H):
        raise ValueError("v must be [batch][n][H][d_v]")
    dv = v.shape[3]
    _need(alpha, "alpha", (torch.float32,), (batch, n, H))
    _need(beta, "beta", (torch.float32,), (batch, n, H))
    _need(parent, "parent", (torch.int32,), (batch, n))
    _need(S0, "S0", (torch.float32,), (batch, H, dk, dv))
    if out is None:
        out = torch.empty((batch, n, H, dv), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), (batch, n, H, dv))
    if status is not None:
        _need(status, "status", (torch.int32,), (batch,))
    args = (_ptr(q), _ptr(k), _ptr(v), _qkv_dtype(q), _ptr(alpha), _ptr(beta), _ptr(parent),
            _ptr(S0), _ptr(out), batch, n, H, dk, dv, _ptr(status), _stream(stream))
    return _issue(name, getattr(lib, name), args,
                  (q, k, v, alpha, beta, parent, S0, out, status), out, prepare)


def verify(q, k, v, alpha, beta, parent, S0, out=None, status=None, stream=None, prepare=False):
    """gdn_tree_verify: fp32 out [batch][n][H][d_v]; S0 is never written.
    prepare=True returns a Launch instead of launching."""
    return _verify_like("gdn_tree_verify", q, k, v, alpha, beta, parent, S0, out, status, stream,
                        prepare)


def branch_verify(q, k, v, alpha, beta, parent, S0, out=None, status=None, stream=None,
                  prepare=False):
    """gdn_branch_verify: the single-branch recurrent baseline, same result
    as verify()."""
    return _verify_like("gdn_branch_verify", q, k, v, alpha, beta, parent, S0, out, status,
                        stream, prepare)


def commit(S, path, path_len, k, v, alpha, beta, parent, status=None, stream=None,
           prepare=False):
    """gdn_tree_commit: advances S [batch][H][d_k][d_v] in place; returns S.
    prepare=True returns a Launch instead of launching."""
    torch = _torch()
    lib = load()
    _need(k, "k", (torch.bfloat16, torch.float32))
    batch, n, H, dk = k.shape
    _need(v, "v", (k.dtype,))
    dv = v.shape[3]
    _need(S, "S", (torch.float32,), (batch, H, dk, dv))
    _need(path, "path", (torch.int32,))
    if path.dim() != 2 or path.shape[0] != batch:
        raise ValueError("path must be [batch][max_path]")
    _need(path_len, "path_len", (torch.int32,), (batch,))
    _need(alpha, "alpha", (torch.float32,), (batch, n, H))
    _need(beta, "beta", (torch.float32,), (batch, n, H))
    _need(parent, "parent", (torch.int32,), (batch, n))
    if status is not None:
        _need(status, "status", (torch.int32,), (batch,))
    args = (_ptr(S), _ptr(path), _ptr(path_len), int(path.shape[1]), _ptr(k), _ptr(v),
            _qkv_dtype(k), _ptr(alpha), _ptr(beta), _ptr(parent), batch, n, H, dk, dv,
            _ptr(status), _stream(stream))
    return _issue("gdn_tree_commit", lib.gdn_tree_commit, args,
                  (S, path, path_len, k, v, alpha, beta, parent, status), S, prepare)


def commit_verify(S, path, path_len, prev, q, k, v, alpha, beta, parent, out=None,
                  status=None, stream=None, prepare=False, u_prev=None, u_out=None):
    """gdn_tree_commit_verify: commit the previous tree's accepted path into S
    (in place), then verify the new tree from the committed S.

    prev = (k_prev, v_prev, alpha_prev, beta_prev, parent_prev): the tensors
    of the tree the path was accepted from.  u_out ([batch][n][H][d_v], fp32
    or fp16) receives the new tree's pseudo-values; u_prev, the previous
    call's u_out on this same S (same dtype), lets the commit skip its
    solve.  Returns out [batch][n][H][d_v] (prepare=True: a Launch instead
    of launching).
    """
    torch = _torch()
    lib = load()
    k_prev, v_prev, alpha_prev, beta_prev, parent_prev = prev
    qk = (torch.bfloat16, torch.float32)
    _need(q, "q", qk)
    batch, n, H, dk = q.shape
    _need(k, "k", (q.dtype,), q.shape)
    _need(v, "v", (q.dtype,))
    if tuple(v.shape[:3]) != (batch, n, H):
        raise ValueError("v must be [batch][n][H][d_v]")
    dv = v.shape[3]
    _need(alpha, "alpha", (torch.float32,), (batch, n, H))
    _need(beta, "beta", (torch.float32,), (batch, n, H))
    _need(parent, "parent", (torch.int32,), (batch, n))
    _need(k_prev, "k_prev", (q.dtype,))
    if k_prev.dim() != 4 or k_prev.shape[0] != batch or tuple(k_prev.shape[2:]) != (H, dk):
        raise ValueError("k_prev must be [batch][n_prev][H][d_k]")
    n_prev = k_prev.shape[1]
    _need(v_prev, "v_prev", (q.dtype,), (batch, n_prev, H, dv))
    _need(alpha_prev, "alpha_prev", (torch.float32,), (batch, n_prev, H))
    _need(beta_prev, "beta_prev", (torch.float32,), (batch, n_prev, H))
    _need(parent_prev, "parent_prev", (torch.int32,), (batch, n_prev))
    udt = (torch.float32, torch.float16)
    if u_prev is not None:
        _need(u_prev, "u_prev", udt, (batch, n_prev, H, dv))
    _need(S, "S", (torch.float32,), (batch, H, dk, dv))
    _need(path, "path", (torch.int32,))
    if path.dim() != 2 or path.shape[0] != batch:
        raise ValueError("path must be [batch][max_path]")
    _need(path_len, "path_len", (torch.int32,), (batch,))
    if out is None:
        out = torch.empty((batch, n, H, dv), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), (batch, n, H, dv))
    if u_out is not None:
        _need(u_out, "u_out", udt, (batch, n, H, dv))
    if u_prev is not None and u_out is not None and u_prev.dtype != u_out.dtype:
        raise ValueError("u_prev and u_out must share a dtype")
    u_given = u_out if u_out is not None else u_prev
    u_dtype = DTYPE_F16 if (u_given is not None and u_given.dtype == torch.float16) else 0
    if status is not None:
        _need(status, "status", (torch.int32,), (batch,))
    args = (_ptr(S), _ptr(path), _ptr(path_len), int(path.shape[1]), _ptr(k_prev),
            _ptr(v_prev), _ptr(alpha_prev), _ptr(beta_prev), _ptr(parent_prev), _ptr(u_prev),
            n_prev, _ptr(q), _ptr(k), _ptr(v), _qkv_dtype(q), _ptr(alpha), _ptr(beta),
            _ptr(parent), _ptr(out), _ptr(u_out), u_dtype, batch, n, H, dk, dv, _ptr(status),
            _stream(stream))
    return _issue("gdn_tree_commit_verify", lib.gdn_tree_commit_verify, args,
                  (S, path, path_len, *prev, u_prev, q, k, v, alpha, beta, parent, out, u_out,
                   status), out, prepare)


def build_tree(cand_logp, cand_tok, root_tok, width, max_depth, stream=None, prepare=False):
    """gdn_tree_build: (parent, token, score, n_built) from a candidate table
    cand_logp fp32 [batch][n][K], cand_tok int32 [batch][n][K]; root_tok
    int32 [batch] or None."""
    torch = _torch()
    lib = load()
    _need(cand_logp, "cand_logp", (torch.float32,))
    if cand_logp.dim() != 3:
        raise ValueError("cand_logp must be [batch][n][K]")
    batch, n, K = cand_logp.shape
    _need(cand_tok, "cand_tok", (torch.int32,), (batch, n, K))
    if root_tok is not None:
        _need(root_tok, "root_tok", (torch.int32,), (batch,))
    dev = cand_logp.device
    parent = torch.empty((batch, n), dtype=torch.int32, device=dev)
    token = torch.empty((batch, n), dtype=torch.int32, device=dev)
    score = torch.empty((batch, n), dtype=torch.float32, device=dev)
    n_built = torch.empty((batch,), dtype=torch.int32, device=dev)
    args = (_ptr(cand_logp), _ptr(cand_tok), _ptr(root_tok), _ptr(parent), _ptr(token),
            _ptr(score), _ptr(n_built), batch, n, K, int(width), int(max_depth), _stream(stream))
    return _issue("gdn_tree_build", lib.gdn_tree_build, args,
                  (cand_logp, cand_tok, root_tok, parent, token, score, n_built),
                  (parent, token, score, n_built), prepare)


def accept(parent, draft_tok, verify_tok, status=None, stream=None, prepare=False):
    """gdn_tree_accept: (accepted, accept_len, bonus_tok), int32 [batch] each."""
    torch = _torch()
    lib = load()
    _need(parent, "parent", (torch.int32,))
    batch, n = parent.shape
    _need(draft_tok, "draft_tok", (torch.int32,), (batch, n))
    _need(verify_tok, "verify_tok", (torch.int32,), (batch, n))
    acc = torch.empty((batch,), dtype=torch.int32, device=parent.device)
    alen = torch.empty((batch,), dtype=torch.int32, device=parent.device)
    bonus = torch.empty((batch,), dtype=torch.int32, device=parent.device)
    if status is not None:
        _need(status, "status", (torch.int32,), (batch,))
    args = (_ptr(parent), _ptr(draft_tok), _ptr(verify_tok), _ptr(acc), _ptr(alen), _ptr(bonus),
            batch, n, _ptr(status), _stream(stream))
    return _issue("gdn_tree_accept", lib.gdn_tree_accept, args,
                  (parent, draft_tok, verify_tok, acc, alen, bonus, status), (acc, alen, bonus),
                  prepare)


def path(parent, accepted, max_path, out=None, path_len=None, status=None, stream=None,
         prepare=False):
    """gdn_tree_path: (path int32 [batch][max_path], path_len int32 [batch])."""
    torch = _torch()
    lib = load()
    _need(parent, "parent", (torch.int32,))
    batch, n = parent.shape
    _need(accepted, "accepted", (torch.int32,), (batch,))
    if out is None:
        out = torch.empty((batch, max_path), dtype=torch.int32, device=parent.device)
    if path_len is None:
        path_len = torch.empty((batch,), dtype=torch.int32, device=parent.device)
    _need(out, "path", (torch.int32,), (batch, max_path))
    _need(path_len, "path_len", (torch.int32,), (batch,))
    if status is not None:
        _need(status, "status", (torch.int32,), (batch,))
    args = (_ptr(parent), _ptr(accepted), _ptr(out), _ptr(path_len), batch, n, int(max_path),
            _ptr(status), _stream(stream))
    return _issue("gdn_tree_path", lib.gdn_tree_path, args,
                  (parent, accepted, out, path_len, status), (out, path_len), prepare)


def index(parent, status=None, stream=None):
    """gdn_tree_index: (depth int32 [batch][n], anc int32 bit patterns [batch][n][ceil(n/32)])."""
    torch = _torch()
    lib = load()
    _need(parent, "parent", (torch.int32,))
    batch, n = parent.shape
    W = (n + 31) // 32
    depth = torch.empty((batch, n), dtype=torch.int32, device=parent.device)
    anc = torch.empty((batch, n, W), dtype=torch.int32, device=parent.device)
    if status is not None:
        _need(status, "status", (torch.int32,), (batch,))
    rc = lib.gdn_tree_index(_ptr(parent), _ptr(depth), _ptr(anc), batch, n, _ptr(status),
                            _stream(stream))
    _check("gdn_tree_index", rc)
    return depth, anc
