"""CPU-side checks of the C ABI: the library loads, exports every entry
point declared in include/gdn_tree.h, and rejects bad arguments on the host
before any launch.  Nothing here reaches a GPU: every call below fails host
validation first (null, misaligned or out-of-range arguments)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_tree_verify_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_tree.h")
FAKE = 0x10000          # an aligned address that is never dereferenced
MISALIGNED = 0x10004


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.lib_path()):
        g.build()
    return g.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gdn_tree_verify", "gdn_branch_verify", "gdn_tree_commit", "gdn_tree_commit_verify",
            "gdn_tree_path", "gdn_tree_accept", "gdn_tree_build",
            "gdn_tree_index", "gdn_status_string", "gdn_tree_abi_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_strings(lib):
    m = re.search(r"#define GDN_TREE_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.gdn_tree_abi_version() == int(m.group(1))
    # the binding's signatures follow the same header version (load() refuses
    # a library of another version)
    assert g.ABI_VERSION == int(m.group(1))
    for code in (0, -1, -2, -3, 5):
        assert isinstance(g.status_string(code), str) and g.status_string(code)


def test_load_refuses_another_abi_version(lib, monkeypatch):
    # a binding that expects another version must not call into this library
    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "ABI_VERSION", lib.gdn_tree_abi_version() + 1)
    with pytest.raises(RuntimeError, match="ABI version"):
        g.load()
    monkeypatch.undo()
    assert g.load() is lib


def _verify(lib, ptr=FAKE, batch=1, n=8, H=1, dk=16, dv=16, dtype=1, null=None, status=None,
            fn="gdn_tree_verify"):
    p = [ptr] * 8
    if null is not None:
        p[null] = None
    return getattr(lib, fn)(p[0], p[1], p[2], dtype, p[3], p[4], p[5], p[6], p[7],
                            batch, n, H, dk, dv, status, None)


@pytest.mark.parametrize("fn", ["gdn_tree_verify", "gdn_branch_verify"])
@pytest.mark.parametrize("null", range(8))
def test_verify_null_pointer(lib, null, fn):
    assert _verify(lib, null=null, fn=fn) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -1), (dict(n=0), -1), (dict(H=0), -1), (dict(dk=0), -1),
    (dict(n=129), -2), (dict(dk=12), -2), (dict(dv=136), -2), (dict(dk=4), -2),
    (dict(dtype=7), -1), (dict(ptr=MISALIGNED), -1), (dict(status=MISALIGNED), -1),
    (dict(batch=1 << 20, H=1 << 12), -2),
])
@pytest.mark.parametrize("fn", ["gdn_tree_verify", "gdn_branch_verify"])
def test_verify_rejects(lib, kw, code, fn):
    assert _verify(lib, fn=fn, **kw) == code


def test_commit_rejects(lib):
    P = FAKE
    ok = dict(max_path=4, batch=1, n=8, H=1, dk=16, dv=16)

    def call(S=P, max_path=4, batch=1, n=8, H=1, dk=16, dv=16, dtype=1):
        return lib.gdn_tree_commit(S, P, P, max_path, P, P, dtype, P, P, P, batch, n, H, dk, dv,
                                   None, None)
    assert call(S=None) == -1
    assert call(max_path=0) == -1
    assert call(n=200) == -2
    assert call(dk=20) == -2
    assert call(S=MISALIGNED) == -1
    assert call(dtype=3) == -1
    del ok


def _commit_verify(lib, null=None, ptr=FAKE, max_path=4, n_prev=8, batch=1, n=8, H=1, dk=16,
                   dv=16, dtype=1, status=None, u_prev=None, u_out=None, u_dtype=0):
    p = [ptr] * 15    # S path path_len k_prev v_prev a_prev b_prev par_prev q k v a b par out
    if null is not None:
        p[null] = None
    return lib.gdn_tree_commit_verify(p[0], p[1], p[2], max_path, p[3], p[4], p[5], p[6], p[7],
                                      u_prev, n_prev, p[8], p[9], p[10], dtype, p[11], p[12],
                                      p[13], p[14], u_out, u_dtype, batch, n, H, dk, dv, status,
                                      None)


@pytest.mark.parametrize("null", range(15))
def test_commit_verify_null_pointer(lib, null):
    assert _commit_verify(lib, null=null) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(max_path=0), -1), (dict(n_prev=0), -1), (dict(n=0), -1), (dict(batch=0), -1),
    (dict(n_prev=129), -2), (dict(n=129), -2), (dict(dk=12), -2), (dict(dv=256), -2),
    (dict(dtype=2), -1), (dict(ptr=MISALIGNED), -1), (dict(status=MISALIGNED), -1),
    (dict(u_prev=MISALIGNED), -1), (dict(u_out=MISALIGNED), -1),
    (dict(u_out=FAKE), -2),        # pseudo-values out need bf16 q/k/v and d = 128
    (dict(u_out=FAKE, u_dtype=2), -2),
    (dict(u_out=FAKE, dtype=0, dk=128, dv=128), -2),   # fp32 q/k/v: no pseudo-values out
    (dict(u_out=FAKE, u_dtype=1), -1),   # pseudo-values are fp32 or fp16
    (dict(u_prev=FAKE, u_dtype=3), -1),
])
def test_commit_verify_rejects(lib, kw, code):
    assert _commit_verify(lib, **kw) == code


def test_path_and_index_reject(lib):
    P = FAKE
    assert lib.gdn_tree_build(None, P, None, P, P, P, None, 1, 8, 4, 2, 4, None) == -1
    assert lib.gdn_tree_build(P, P, None, P, P, P, None, 1, 8, 4, 0, 4, None) == -1
    assert lib.gdn_tree_build(P, P, None, P, P, P, None, 1, 8, 4, 2, -1, None) == -1
    assert lib.gdn_tree_build(P, P, None, P, P, P, None, 1, 8, 33, 2, 4, None) == -2
    assert lib.gdn_tree_build(P, P, None, P, P, P, None, 1, 129, 4, 2, 4, None) == -2
    assert lib.gdn_tree_build(P, P, MISALIGNED, P, P, P, None, 1, 8, 4, 2, 4, None) == -1
    assert lib.gdn_tree_accept(None, P, P, P, None, None, 1, 8, None, None) == -1
    assert lib.gdn_tree_accept(P, P, P, None, None, None, 1, 8, None, None) == -1
    assert lib.gdn_tree_accept(P, P, P, P, None, None, 0, 8, None, None) == -1
    assert lib.gdn_tree_accept(P, P, P, P, None, None, 1, 129, None, None) == -2
    assert lib.gdn_tree_accept(P, P, P, P, MISALIGNED, None, 1, 8, None, None) == -1
    assert lib.gdn_tree_path(None, P, P, P, 1, 8, 4, None, None) == -1
    assert lib.gdn_tree_path(P, P, P, P, 1, 8, 0, None, None) == -1
    assert lib.gdn_tree_path(P, P, P, P, 1, 129, 4, None, None) == -2
    assert lib.gdn_tree_path(P, P, P, MISALIGNED, 1, 8, 4, None, None) == -1
    assert lib.gdn_tree_index(P, None, P, 1, 8, None, None) == -1
    assert lib.gdn_tree_index(P, P, P, 0, 8, None, None) == -1
    assert lib.gdn_tree_index(P, P, P, 1, 300, None, None) == -2


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 8, 1, 16)
    with pytest.raises(ValueError):
        g.verify(q, q, q, torch.zeros(1, 8, 1), torch.zeros(1, 8, 1),
                 torch.zeros(1, 8, dtype=torch.int32), torch.zeros(1, 1, 16, 16))


def test_product_package_does_not_import_oracle():
    """the product path never reaches the test oracle"""
    pkg = os.path.dirname(g.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "gdn_oracle" not in text and "liboracle" not in text, f
