"""fp64 CPU oracle for GDN tree verification -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never does, and shares no code with it.

``gdn_oracle.c`` replays the Gated DeltaNet recurrence of the Trees from
Marginals technical summary (Methodology, "3. Rollback-Free Tree Verification
for GDN") from the prefix state S0 along every root-to-node path in fp64; see
that file's header for the exact definition and index conventions.  This
module compiles it with gcc and calls it through ctypes.

Every function here is pinned by ``tests/test_oracle_pins.py``; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
# The mutation tests point this at a deliberately broken copy of the oracle
# to show that the pins catch planted mistakes.
_OVERRIDE = os.environ.get("GDN_ORACLE_LIB_OVERRIDE")

_ERRORS = {-1: "bad dims", -2: "invalid tree (parent[i] outside [-1, i-1])",
           -3: "invalid accepted node", -4: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with gcc (fp contraction off: fixed fp64 rounding)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
           *extra, "-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


_lib_cache = {}


def load(path: str = None):
    if path is None:
        path = _OVERRIDE or _LIB
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path) or (path == _LIB and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        if path != _LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    up = ctypes.POINTER(ctypes.c_uint32)
    ci = ctypes.c_int
    lib.oracle_verify.argtypes = [ci] * 6 + [dp] * 5 + [ip, dp, dp, ci, ci]
    lib.oracle_verify.restype = ci
    lib.oracle_commit.argtypes = [ci] * 6 + [dp] * 4 + [ip, dp, ip, dp, ci]
    lib.oracle_commit.restype = ci
    lib.oracle_ancestors.argtypes = [ci, ci, ip, up, ip]
    lib.oracle_ancestors.restype = ci
    lib.oracle_check_tree.argtypes = [ci, ci, ip]
    lib.oracle_check_tree.restype = ci
    _lib_cache[path] = lib
    return lib


def _d(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _check(rc: int):
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, f"oracle error {rc}"))


MAX_THREADS = 16


def default_threads() -> int:
    """Worker threads when none are given: OMP_NUM_THREADS if set, else the
    CPUs this process may run on, at most MAX_THREADS."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = int(env)
    else:
        try:
            n = len(os.sched_getaffinity(0))
        except AttributeError:
            n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _threads(n):
    return int(n) if n else default_threads()


def verify(q, k, v, g, beta, parent, S0, memo: bool = True, threads=None, lib=None) -> np.ndarray:
    """o[B][N][Hv][dv] (float64): each node's output after its own update,
    the recurrence run from S0 along the node's root..node path."""
    lib = lib or load()
    q, k, v, g, beta, S0 = map(_d, (q, k, v, g, beta, S0))
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    B, N, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    o = np.zeros((B, N, Hv, dv), dtype=np.float64)
    rc = lib.oracle_verify(B, N, Hk, Hv, dk, dv, _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                           _ptr(v, ctypes.c_double), _ptr(g, ctypes.c_double),
                           _ptr(beta, ctypes.c_double), _ptr(parent, ctypes.c_int32),
                           _ptr(S0, ctypes.c_double), _ptr(o, ctypes.c_double),
                           1 if memo else 0, _threads(threads))
    _check(rc)
    return o


def commit(k, v, g, beta, parent, S0, accepted, threads=None, lib=None) -> np.ndarray:
    """S_new[B][Hv][dv][dk] (float64): the state the recurrence reaches at
    accepted[b] (S0 where accepted[b] == -1)."""
    lib = lib or load()
    k, v, g, beta, S0 = map(_d, (k, v, g, beta, S0))
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    accepted = np.ascontiguousarray(accepted, dtype=np.int32)
    B, N, Hk, dk = k.shape
    Hv, dv = v.shape[2], v.shape[3]
    out = np.zeros((B, Hv, dv, dk), dtype=np.float64)
    rc = lib.oracle_commit(B, N, Hk, Hv, dk, dv, _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                           _ptr(g, ctypes.c_double), _ptr(beta, ctypes.c_double),
                           _ptr(parent, ctypes.c_int32), _ptr(S0, ctypes.c_double),
                           _ptr(accepted, ctypes.c_int32), _ptr(out, ctypes.c_double),
                           _threads(threads))
    _check(rc)
    return out


def ancestors(parent, lib=None):
    """(anc, depth): anc[B][N][ceil(N/32)] uint32 bit rows, bit s of row i set
    iff s is on the root..i path (i included); depth[B][N] = path length."""
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    B, N = parent.shape
    W = (N + 31) // 32
    anc = np.zeros((B, N, max(W, 1)), dtype=np.uint32)
    depth = np.zeros((B, N), dtype=np.int32)
    _check(lib.oracle_ancestors(B, N, _ptr(parent, ctypes.c_int32), _ptr(anc, ctypes.c_uint32),
                                _ptr(depth, ctypes.c_int32)))
    return anc[:, :, :W], depth


def check_tree(parent, lib=None) -> bool:
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    B, N = parent.shape
    return lib.oracle_check_tree(B, N, _ptr(parent, ctypes.c_int32)) == 0


def verify_inputs(inp: dict, **kw) -> np.ndarray:
    """verify() on a dict produced by the seeded input generators."""
    return verify(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["parent"], inp["S0"], **kw)


def commit_inputs(inp: dict, accepted=None, **kw) -> np.ndarray:
    acc = inp["accepted"] if accepted is None else accepted
    return commit(inp["k"], inp["v"], inp["g"], inp["beta"], inp["parent"], inp["S0"], acc, **kw)
