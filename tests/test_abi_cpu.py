"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_tree_gdn_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_tree.h")

FAKE = 0x10000  # never dereferenced: every call below fails before touching it


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn_tree.so is not built: run __graft_entry__.build()")
    return gdn.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def dims(**kw):
    d = dict(B=2, N=16, H_k=2, H_v=4, d_k=128, d_v=128, qkv_dtype=gdn.GDN_BF16)
    d.update(kw)
    return gdn.Dims(**d)


def make_ctx(lib, d):
    h = ctypes.c_void_p()
    n = lib.gdn_tree_workspace_bytes(ctypes.byref(d))
    rc = lib.gdn_ctx_create(ctypes.byref(d), FAKE, n, ctypes.byref(h))
    return rc, h


def test_status_strings(lib):
    for code, name in enumerate(gdn.STATUS):
        assert lib.gdn_status_string(code).decode() == name


def test_workspace_bytes(lib):
    n = lib.gdn_tree_workspace_bytes(ctypes.byref(dims(B=1000)))
    assert n >= 8000 and n % 256 == 0
    assert lib.gdn_tree_workspace_bytes(None) == 0


@pytest.mark.parametrize("B,N,H_v", [(64, 256, 32), (3, 129, 4), (1, 200, 1)])
def test_workspace_holds_the_two_launch_intermediate(lib, B, N, H_v):
    """trees of more than 128 nodes: the verdict words plus, per (sequence,
    value head), 24 N pair values and N gammas, and per sequence a 2-byte
    place per pair and N + 1 offsets; trees of at most 128 nodes: only the
    verdict words"""
    d = dims(B=B, N=N, H_k=1, H_v=H_v)
    n = lib.gdn_tree_workspace_bytes(ctypes.byref(d))
    need = 8 * B + 4 * (24 * N + N) * H_v * B + 2 * 24 * N * B + 4 * (N + 1) * B + 4 * B
    assert n % 256 == 0 and need <= n <= need + 8 * 256
    small = dims(B=B, N=128, H_k=1, H_v=H_v)
    assert lib.gdn_tree_workspace_bytes(ctypes.byref(small)) == max(256, -(-8 * B // 256) * 256)


@pytest.mark.parametrize("kw,code", [
    (dict(N=257), "GDN_ERR_SHAPE"), (dict(N=-1), "GDN_ERR_SHAPE"), (dict(B=-3), "GDN_ERR_SHAPE"),
    (dict(H_v=3), "GDN_ERR_SHAPE"), (dict(H_k=0), "GDN_ERR_SHAPE"), (dict(d_k=96), "GDN_ERR_SHAPE"),
    (dict(d_v=256), "GDN_ERR_SHAPE"), (dict(qkv_dtype=7), "GDN_ERR_DTYPE"),
])
def test_bad_dims_rejected(lib, kw, code):
    rc, h = make_ctx(lib, dims(**kw))
    assert gdn.STATUS[rc] == code
    assert lib.gdn_last_error().decode()
    assert not h.value


def test_workspace_checks(lib):
    d = dims()
    h = ctypes.c_void_p()
    assert gdn.STATUS[lib.gdn_ctx_create(ctypes.byref(d), None, 4096, ctypes.byref(h))] == "GDN_ERR_WORKSPACE"
    assert gdn.STATUS[lib.gdn_ctx_create(ctypes.byref(d), FAKE, 4, ctypes.byref(h))] == "GDN_ERR_WORKSPACE"
    assert gdn.STATUS[lib.gdn_ctx_create(ctypes.byref(d), FAKE + 16, 4096, ctypes.byref(h))] == "GDN_ERR_ALIGN"
    assert gdn.STATUS[lib.gdn_ctx_create(ctypes.byref(d), FAKE, 4096, None)] == "GDN_ERR_NULL"


def verify_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, parent=FAKE, S0=FAKE, o=FAKE)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "g", "beta", "parent", "S0", "o")]


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "parent", "S0", "o"])
def test_verify_null_and_misaligned(lib, name):
    rc, h = make_ctx(lib, dims())
    assert rc == 0
    try:
        rc = lib.gdn_tree_verify(h, *verify_args(**{name: None}), None)
        assert gdn.STATUS[rc] == "GDN_ERR_NULL"
        assert name in lib.gdn_last_error().decode()
        rc = lib.gdn_tree_verify(h, *verify_args(**{name: FAKE + 4}), None)
        assert gdn.STATUS[rc] == "GDN_ERR_ALIGN"
    finally:
        lib.gdn_ctx_destroy(h)


def test_commit_without_verify(lib):
    rc, h = make_ctx(lib, dims())
    assert rc == 0
    try:
        assert gdn.STATUS[lib.gdn_commit_path(h, FAKE, FAKE, None)] == "GDN_ERR_STATE"
        # a verify that failed its checks does not arm the commit either
        lib.gdn_tree_verify(h, *verify_args(q=None), None)
        assert gdn.STATUS[lib.gdn_commit_path(h, FAKE, FAKE, None)] == "GDN_ERR_STATE"
    finally:
        lib.gdn_ctx_destroy(h)


def test_empty_batch_is_noop(lib):
    for d in (dims(B=0), dims(N=0)):
        rc, h = make_ctx(lib, d)
        assert rc == 0
        try:
            assert lib.gdn_tree_verify(h, *verify_args(q=None, o=None), None) == 0
        finally:
            lib.gdn_ctx_destroy(h)


def test_null_ctx(lib):
    assert gdn.STATUS[lib.gdn_tree_verify(None, *verify_args(), None)] == "GDN_ERR_NULL"
    assert gdn.STATUS[lib.gdn_commit_path(None, FAKE, FAKE, None)] == "GDN_ERR_NULL"
    assert gdn.STATUS[lib.gdn_ctx_status(None, None)] == "GDN_ERR_NULL"
    assert lib.gdn_ctx_destroy(None) == 0


def test_ancestors_arg_checks(lib):
    d = dims(N=300)
    assert gdn.STATUS[lib.gdn_tree_ancestors(ctypes.byref(d), FAKE, FAKE, FAKE, None, None)] == "GDN_ERR_SHAPE"
    d = dims()
    assert gdn.STATUS[lib.gdn_tree_ancestors(ctypes.byref(d), None, FAKE, FAKE, None, None)] == "GDN_ERR_NULL"
    assert gdn.STATUS[lib.gdn_tree_ancestors(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 4, None)] == "GDN_ERR_ALIGN"
    assert lib.gdn_tree_ancestors(ctypes.byref(dims(B=0)), None, None, None, None, None) == 0


def test_python_binding_has_no_cpu_fallback():
    """the binding never imports the oracle and has no CPU compute path"""
    src = open(os.path.join(ROOT, "gated_deltanet_tree_gdn_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("oracle is", "")
    assert "numpy" not in src


def test_accept_path_arg_checks(lib):
    d = dims(N=300)
    assert gdn.STATUS[lib.gdn_accept_path(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None)] == "GDN_ERR_SHAPE"
    d = dims()
    assert gdn.STATUS[lib.gdn_accept_path(None, FAKE, FAKE, FAKE, FAKE, None, None, None)] == "GDN_ERR_NULL"
    for i in range(4):
        args = [FAKE] * 4
        args[i] = None
        assert gdn.STATUS[lib.gdn_accept_path(ctypes.byref(d), *args, None, None, None)] == "GDN_ERR_NULL"
        args[i] = FAKE + 4
        assert gdn.STATUS[lib.gdn_accept_path(ctypes.byref(d), *args, None, None, None)] == "GDN_ERR_ALIGN"
    assert gdn.STATUS[lib.gdn_accept_path(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE + 8, None, None)] == "GDN_ERR_ALIGN"
    assert lib.gdn_accept_path(ctypes.byref(dims(B=0)), None, None, None, None, None, None, None) == 0


def test_tree_build_arg_checks(lib):
    d = dims()
    ok = (8, 4, 16, FAKE, FAKE, FAKE, None, None, None, None, None)
    for bad in ((0,) + ok[1:], (33,) + ok[1:], ok[:1] + (0,) + ok[2:], ok[:2] + (0,) + ok[3:]):
        assert gdn.STATUS[lib.gdn_tree_build(ctypes.byref(d), *bad)] == "GDN_ERR_SHAPE"
    assert gdn.STATUS[lib.gdn_tree_build(ctypes.byref(dims(N=257)), *ok)] == "GDN_ERR_SHAPE"
    for i in (3, 4, 5):
        args = list(ok)
        args[i] = None
        assert gdn.STATUS[lib.gdn_tree_build(ctypes.byref(d), *args)] == "GDN_ERR_NULL"
        args[i] = FAKE + 4
        assert gdn.STATUS[lib.gdn_tree_build(ctypes.byref(d), *args)] == "GDN_ERR_ALIGN"
    assert lib.gdn_tree_build(ctypes.byref(dims(N=0)), *ok) == 0


def test_verify_static_arg_checks(lib):
    """the allocation-free verify rejects B beyond its fixed scratch, bad
    shapes, NULL and misaligned pointers, all on the host"""
    ptrs = [FAKE] * 8 + [None]
    limit = int(re.search(r"#define GDN_STATIC_MAX_B (\d+)", open(HEADER).read()).group(1))
    assert gdn.STATUS[lib.gdn_tree_verify_static(ctypes.byref(dims(B=limit + 1)), *ptrs)] == "GDN_ERR_SHAPE"
    assert "at most %d" % limit in lib.gdn_last_error().decode()
    assert gdn.STATUS[lib.gdn_tree_verify_static(None, *ptrs)] == "GDN_ERR_NULL"
    for bad in (dict(N=257), dict(H_v=3), dict(d_k=96), dict(B=-1)):
        assert gdn.STATUS[lib.gdn_tree_verify_static(ctypes.byref(dims(**bad)), *ptrs)] == "GDN_ERR_SHAPE"
    assert gdn.STATUS[lib.gdn_tree_verify_static(ctypes.byref(dims(qkv_dtype=7)), *ptrs)] == "GDN_ERR_DTYPE"
    for i in range(8):
        args = list(ptrs)
        args[i] = None
        assert gdn.STATUS[lib.gdn_tree_verify_static(ctypes.byref(dims()), *args)] == "GDN_ERR_NULL"
        args[i] = FAKE + 8
        assert gdn.STATUS[lib.gdn_tree_verify_static(ctypes.byref(dims()), *args)] == "GDN_ERR_ALIGN"
    assert lib.gdn_tree_verify_static(ctypes.byref(dims(B=0)), *ptrs) == 0
    assert lib.gdn_tree_verify_static(ctypes.byref(dims(N=0)), *ptrs) == 0
