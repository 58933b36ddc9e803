"""Seeded synthetic inputs for GDN tree verification.

This module only *creates data*: proposal trees and the tensors a Gated
DeltaNet layer hands to tree verification.  It holds none of the method's
arithmetic (no recurrence, no decay products, no solve), so both the fp64
oracle and the HIP path may consume what it produces.

Workload recipe (the pages give no data; these stand in for the draft trees a
27B verifier sees at "tree size 128", Trees-from-Marginals technical summary,
Experimental Results):

* RNG: ``numpy.random.default_rng([seed, layer])``; draws happen in the fixed
  order parent -> q -> k -> v -> g -> beta -> S0 -> accepted.
* q, k ~ N(0, 1) in fp32, L2-normalised over d_k in fp32, then rounded to
  bf16 (round-to-nearest-even) unless the dtype is fp32.  v ~ N(0, 1) rounded
  the same way.
* beta = sigmoid(N(0, 1)), g = -softplus(N(0, 1)) (a log-decay, g <= 0),
  S0 = 0.02 * N(0, 1); all fp32.
* accepted[b] ~ U{0 .. N-1}.
* Trees (int32 parent arrays in topological order, -1 = child of the prefix
  state): ``uniform`` (parent[i] ~ U{0..i-1}), ``chain`` (parent[i] = i-1) and
  ``best_first`` (a w = 1 reading of the best-first draft-tree construction,
  Technical Summary, Methodology, 2. Tree Construction; see
  :func:`tree_best_first`).

Layouts (row-major, C order):
  q, k    [B][N][H_k][d_k]
  v       [B][N][H_v][d_v]
  g, beta [B][N][H_v]
  parent  [B][N]
  S0      [B][H_v][d_v][d_k]   (state maps a key to a value: o = S q)
  accepted[B]
"""
from __future__ import annotations

import dataclasses
import heapq
from typing import Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "rng_for", "tree_uniform", "tree_chain", "tree_best_first",
    "round_bf16_bits", "bf16_bits_to_f32", "make_inputs", "make_inputs_device", "tree_stats",
    "to_device", "shrink", "make_draft_tokens", "make_candidate_logp",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape and tree recipe of one workload."""
    name: str
    B: int
    N: int
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    tree: str               # "uniform" | "chain" | "best_first"
    max_depth: int = 0      # depth cap for best_first (root has depth 1)
    dtype: str = "bf16"     # dtype of q, k, v: "bf16" | "f32"
    layers: int = 1         # independent layers (tensors per layer; tree shared)
    commit: bool = False    # draw accepted[] too


# Workloads, each named for its shape and tree.
CONFIGS = {
    "tiny_f32": Config("tiny_f32", B=1, N=8, H_k=1, H_v=1, d_k=64, d_v=64,
                       tree="uniform", dtype="f32"),
    "chain64": Config("chain64", B=1, N=64, H_k=16, H_v=16, d_k=128, d_v=128,
                      tree="chain"),
    "bestfirst128": Config("bestfirst128", B=1, N=128, H_k=16, H_v=32, d_k=128, d_v=128,
                           tree="best_first", max_depth=16),
    "batched_commit": Config("batched_commit", B=32, N=64, H_k=32, H_v=32, d_k=128, d_v=128,
                             tree="best_first", max_depth=16, commit=True),
    "stress48": Config("stress48", B=64, N=256, H_k=16, H_v=32, d_k=128, d_v=128,
                       tree="best_first", max_depth=24, layers=48),
    "bestfirst_b32n128": Config("bestfirst_b32n128", B=32, N=128, H_k=16, H_v=32, d_k=128, d_v=128,
                       tree="best_first", max_depth=16),
}


def rng_for(seed: int = 0, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, layer])


# ----------------------------------------------------------------------------
# Trees
# ----------------------------------------------------------------------------

def tree_uniform(rng: np.random.Generator, B: int, N: int) -> np.ndarray:
    """parent[0] = -1, parent[i] ~ U{0..i-1}."""
    par = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        if N == 0:
            continue
        par[b, 0] = -1
        if N > 1:
            par[b, 1:] = rng.integers(0, np.arange(1, N))
    return par


def tree_chain(B: int, N: int) -> np.ndarray:
    """parent[i] = i - 1: one branch, the plain token-by-token sequence."""
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    return par.reshape(B, N)


_ZIPF_S = 1.2
_ZIPF_RANKS = 8


def _one_best_first(rng: np.random.Generator, N: int, max_depth: int) -> np.ndarray:
    """One best-first-shaped tree of N nodes (w = 1 expansion per step).

    Root 0 scores 0.  Repeatedly pop the best-scoring unexpanded node (ties go
    to the lower index); a node at the depth cap is not expanded.  Otherwise a
    branching factor c is drawn from a Zipf(1.2) law truncated to ranks 1..8
    and min(c, N - count) children are appended in rank order (so indices stay
    topological); child r scores score(parent) + log u_(r) with the u's sorted
    in descending order.  If the heap runs dry before N nodes exist, every
    node below the cap that has fewer than 8 children is pushed again; a node
    expanded a second time receives at most 8 children in all, so no node
    ever has more than 8.
    """
    ranks = np.arange(1, _ZIPF_RANKS + 1, dtype=np.float64)
    p = ranks ** (-_ZIPF_S)
    p /= p.sum()
    parent = np.full(N, -1, dtype=np.int32)
    if N == 0:
        return parent
    depth = [1]
    score = [0.0]
    kids = [0]
    heap = [(-0.0, 0)]
    count = 1
    while count < N:
        if not heap:
            heap = [(-score[i], i) for i in range(count) if depth[i] < max_depth and kids[i] < _ZIPF_RANKS]
            heapq.heapify(heap)
            if not heap:
                raise ValueError("depth cap too small for N nodes")
        _, node = heapq.heappop(heap)
        if depth[node] >= max_depth or kids[node] >= _ZIPF_RANKS:
            continue
        c = int(rng.choice(_ZIPF_RANKS, p=p)) + 1
        u = np.sort(rng.random(c))[::-1]
        m = min(c, _ZIPF_RANKS - kids[node], N - count)
        kids[node] += m
        for r in range(m):
            parent[count] = node
            depth.append(depth[node] + 1)
            kids.append(0)
            score.append(score[node] + float(np.log(u[r])))
            heapq.heappush(heap, (-score[count], count))
            count += 1
    return parent


def tree_best_first(rng: np.random.Generator, B: int, N: int, max_depth: int) -> np.ndarray:
    """B independent best-first-shaped trees (see :func:`_one_best_first`)."""
    return np.stack([_one_best_first(rng, N, max_depth) for _ in range(B)]).astype(np.int32).reshape(B, N)


def tree_stats(parent: np.ndarray) -> dict:
    """Mean strict-ancestor count and maximum depth (root depth 1): data only."""
    B, N = parent.shape
    depth = np.zeros((B, N), dtype=np.int64)
    for b in range(B):
        for i in range(N):
            p = parent[b, i]
            depth[b, i] = 1 if p < 0 else depth[b, p] + 1
    return {"mean_strict_ancestors": float((depth - 1).mean()) if N else 0.0,
            "max_depth": int(depth.max()) if N else 0}


# ----------------------------------------------------------------------------
# bf16 encoding (data representation, not arithmetic of the method)
# ----------------------------------------------------------------------------

def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs cannot overflow 32 bits here (largest is 0xFF7FFFFF + 0x8000)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Tensors
# ----------------------------------------------------------------------------

def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    return (x / n).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (np.float32(1) / (np.float32(1) + np.exp(-x))).astype(np.float32)


def make_tree(cfg: Config, rng: np.random.Generator, B: Optional[int] = None) -> np.ndarray:
    B = cfg.B if B is None else B
    if cfg.tree == "uniform":
        return tree_uniform(rng, B, cfg.N)
    if cfg.tree == "chain":
        return tree_chain(B, cfg.N)
    if cfg.tree == "best_first":
        return tree_best_first(rng, B, cfg.N, cfg.max_depth)
    raise ValueError(f"unknown tree recipe {cfg.tree!r}")


def make_inputs(cfg: Config, seed: int = 0, layer: int = 0, parent: Optional[np.ndarray] = None) -> dict:
    """All tensors of one layer of ``cfg`` as numpy arrays.

    Returns a dict with ``parent`` (int32), ``q``, ``k``, ``v`` (float32 values;
    exactly bf16-representable when cfg.dtype == "bf16"), ``q_bits``,
    ``k_bits``, ``v_bits`` (uint16, bf16 only), ``g``, ``beta``, ``S0``
    (float32) and ``accepted`` (int32, when cfg.commit).  A ``parent`` passed
    in (a tree shared across layers) replaces the drawn one; the draw still
    happens so the tensor stream does not depend on it.
    """
    rng = rng_for(seed, layer)
    B, N, Hk, Hv, dk, dv = cfg.B, cfg.N, cfg.H_k, cfg.H_v, cfg.d_k, cfg.d_v
    drawn = make_tree(cfg, rng)
    par = drawn if parent is None else np.ascontiguousarray(parent, dtype=np.int32)
    q = _l2_normalise(rng.standard_normal((B, N, Hk, dk), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal((B, N, Hk, dk), dtype=np.float32))
    v = rng.standard_normal((B, N, Hv, dv), dtype=np.float32)
    g = -_softplus(rng.standard_normal((B, N, Hv), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((B, N, Hv), dtype=np.float32))
    S0 = (np.float32(0.02) * rng.standard_normal((B, Hv, dv, dk), dtype=np.float32)).astype(np.float32)
    out = {"parent": par, "g": g, "beta": beta, "S0": S0, "cfg": cfg}
    if cfg.dtype == "bf16":
        for name, x in (("q", q), ("k", k), ("v", v)):
            bits = round_bf16_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
    elif cfg.dtype == "f32":
        out.update(q=q, k=k, v=v)
    else:
        raise ValueError(cfg.dtype)
    if cfg.commit:
        out["accepted"] = rng.integers(0, N, size=B).astype(np.int32)
    return out


def shrink(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller test sizes)."""
    return dataclasses.replace(cfg, **kw)


def make_inputs_device(cfg: Config, seed: int = 0, layer: int = 0, parent: Optional[np.ndarray] = None,
                       device="cuda"):
    """The same recipe drawn on the device with torch's generator (for the
    48-layer stress workload, where host generation would dominate).

    Values follow the distributions of :func:`make_inputs` but not its exact
    numbers.  Returns torch tensors: q, k, v (bf16 or fp32), g, beta, S0
    (fp32), parent (int32; the given shared tree, else one drawn with numpy).
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((int(seed) * 1_000_003 + int(layer)) & 0x7FFFFFFFFFFFFFFF)
    B, N, Hk, Hv, dk, dv = cfg.B, cfg.N, cfg.H_k, cfg.H_v, cfg.d_k, cfg.d_v
    if parent is None:
        parent = make_tree(cfg, rng_for(seed, layer))
    par = torch.from_numpy(np.ascontiguousarray(parent, dtype=np.int32)).to(device)

    def randn(*shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    q = randn(B, N, Hk, dk)
    q = q / q.norm(dim=-1, keepdim=True)
    k = randn(B, N, Hk, dk)
    k = k / k.norm(dim=-1, keepdim=True)
    v = randn(B, N, Hv, dv)
    g = -torch.nn.functional.softplus(randn(B, N, Hv))
    beta = torch.sigmoid(randn(B, N, Hv))
    S0 = 0.02 * randn(B, Hv, dv, dk)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return {"parent": par, "q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous(),
            "g": g.contiguous(), "beta": beta.contiguous(), "S0": S0.contiguous(), "cfg": cfg}


def to_device(inp: dict, device="cuda") -> dict:
    """Host arrays from :func:`make_inputs` as torch tensors on ``device``
    (bf16 tensors are rebuilt from the exact bit patterns)."""
    import torch

    out = {}
    for name in ("q", "k", "v"):
        if name + "_bits" in inp:
            t = torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(inp[name], dtype=np.float32))
        out[name] = t.to(device).contiguous()
    for name in ("g", "beta", "S0"):
        out[name] = torch.from_numpy(np.ascontiguousarray(inp[name], dtype=np.float32)).to(device)
    out["parent"] = torch.from_numpy(np.ascontiguousarray(inp["parent"], dtype=np.int32)).to(device)
    if "accepted" in inp:
        out["accepted"] = torch.from_numpy(np.ascontiguousarray(inp["accepted"], dtype=np.int32)).to(device)
    return out


# ----------------------------------------------------------------------------
# Tokens and candidate scores for the steps around verification
# ----------------------------------------------------------------------------

def make_draft_tokens(parent: np.ndarray, rng: np.random.Generator, vocab: int = 32000,
                      p_match: float = 0.8):
    """Synthetic drafted tokens and verifier choices for a batch of trees.

    draft_token [B][N]: each node's token; the children of one node draw
    distinct tokens (a drafter proposes distinct continuations).
    target_token [B][N+1]: the verifier's choice after the prefix (index 0)
    and after node i (index i + 1).  With probability p_match it is the token
    of one of that context's children, the k-th child (in index order) picked
    with weight 1 / (k + 1); otherwise a token none of the children drafted.
    """
    parent = np.asarray(parent)
    B, N = parent.shape
    draft = np.zeros((B, N), dtype=np.int32)
    target = np.zeros((B, N + 1), dtype=np.int32)
    for b in range(B):
        kids = {c: [] for c in range(-1, N)}
        for i in range(N):
            kids[int(parent[b, i])].append(i)
        for c, ch in kids.items():
            if ch:
                draft[b, ch] = rng.choice(vocab, size=len(ch), replace=False)
        for c, ch in kids.items():
            if ch and rng.random() < p_match:
                wts = 1.0 / np.arange(1, len(ch) + 1)
                target[b, c + 1] = draft[b, ch[int(rng.choice(len(ch), p=wts / wts.sum()))]]
            else:
                taken = set(int(draft[b, i]) for i in ch)
                t = int(rng.integers(vocab))
                while t in taken:
                    t = int(rng.integers(vocab))
                target[b, c + 1] = t
    return draft, target


def make_candidate_logp(rng: np.random.Generator, B: int, N: int, C: int = 8, alpha: float = 0.3):
    """Synthetic drafter scores for tree construction: root_logp [B][C] and
    node_logp [B][N][C], each row the log of a Dirichlet(alpha) draw over C
    candidates sorted best first (fp32; probabilities below 1e-30 are clipped
    so every log-probability is finite)."""
    p = rng.dirichlet(np.full(C, alpha), size=(B, N + 1))
    p = -np.sort(-p, axis=-1)
    logp = np.log(np.maximum(p, 1e-30)).astype(np.float32)
    return np.ascontiguousarray(logp[:, 0]), np.ascontiguousarray(logp[:, 1:])
