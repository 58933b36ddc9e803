"""Plain host references for the two steps around tree verification --
TEST INFRASTRUCTURE ONLY (used by tests/, never by the product path).

* :func:`tree_build` -- the draft-tree construction upstream of verification:
  a best-first search over candidate continuations that takes the top-w
  candidates of the heap at a time and expands them together, so a tree of
  N nodes needs about ceil(N / w) sequential expansion steps (Trees from
  Marginals technical summary, Methodology, "2. Tree Construction", which
  modifies DySpec's best-first construction this way; wispaper.ai page,
  Methodology, "Dynamic Tree Construction").
* :func:`accept_path` -- the accepted branch the delayed commit needs
  (technical summary, Methodology, "3. Rollback-Free Tree Verification for
  GDN": the state is committed once the accepted branch is known;
  Experimental Results: mean acceptance length).  The pages do not print the
  acceptance rule; the reading used is greedy matching from the root, the
  rule of lossless greedy speculative decoding.

Both are written as the plain sequential procedure, with Python's heapq and
loops; every integer result is exact and every float is an fp32 sum formed
in the same order as the definition states.
"""
from __future__ import annotations

import heapq

import numpy as np


class DraftError(ValueError):
    pass


def _check_parent(parent_row):
    for i, p in enumerate(parent_row):
        if p < -1 or p >= i:
            raise DraftError(f"parent[{i}] = {p} is outside [-1, {i - 1}]")


def accept_path(parent, draft_token, target_token):
    """Greedy acceptance walk, per sequence b.

    Start at the prefix (node -1).  The verifier's choice after the current
    node c is target_token[b][c + 1] (index 0 is its choice after the prefix
    itself).  Among the children of c (the nodes i with parent[b][i] == c),
    find those whose draft token equals that choice; if there are several,
    the lowest index wins.  Move to it and repeat; stop when no child
    matches.  Returns (accepted[B], accept_len[B]): the last node reached
    (-1 if even the first step fails) and the number of drafted tokens
    accepted, which is that node's depth.
    """
    parent = np.asarray(parent, dtype=np.int64)
    draft_token = np.asarray(draft_token, dtype=np.int64)
    target_token = np.asarray(target_token, dtype=np.int64)
    B, N = parent.shape
    if draft_token.shape != (B, N) or target_token.shape != (B, N + 1):
        raise DraftError("draft_token must be [B][N] and target_token [B][N+1]")
    accepted = np.full(B, -1, dtype=np.int32)
    length = np.zeros(B, dtype=np.int32)
    for b in range(B):
        _check_parent(parent[b])
        cur, n = -1, 0
        while True:
            want = target_token[b, cur + 1]
            nxt = -1
            for i in range(N):
                if parent[b, i] == cur and draft_token[b, i] == want:
                    nxt = i
                    break
            if nxt < 0:
                break
            cur, n = nxt, n + 1
        accepted[b], length[b] = cur, n
    return accepted, length


def tree_build(root_logp, node_logp, N, w, max_depth):
    """Top-w best-first draft-tree construction, per sequence b.

    The candidate heap starts with the prefix's candidate continuations,
    candidate r scoring root_logp[b][r] (a log-probability).  Each step pops
    the w best candidates (fewer if the tree is nearly full or the heap runs
    short); ties go to the lower parent index (the prefix, -1, first), then
    to the lower candidate rank.  The popped candidates become nodes count,
    count+1, ... in the order popped, so every node follows its parent.  Once
    the step's nodes exist they are expanded together: node j's candidate r
    scores score[j] + node_logp[b][j][r] (an fp32 sum), and is pushed unless
    node j sits at the depth cap (the prefix's children have depth 1).

    Each row of root_logp and node_logp must be non-increasing (a drafter's
    top-K list, best first).

    Returns (parent [B][N] int32, rank [B][N] int32, score [B][N] float32,
    steps [B] int32).
    """
    root_logp = np.asarray(root_logp, dtype=np.float32)
    node_logp = np.asarray(node_logp, dtype=np.float32)
    B, C = root_logp.shape
    if node_logp.shape != (B, N, C):
        raise DraftError("node_logp must be [B][N][C] with C = root_logp.shape[1]")
    if w < 1 or max_depth < 1 or C < 1:
        raise DraftError("w, max_depth and the candidate count must be >= 1")
    for rows in (root_logp, node_logp.reshape(-1, C)):
        if np.any(rows[..., 1:] > rows[..., :-1]):
            raise DraftError("candidate log-probabilities must be non-increasing in rank")
    parent = np.full((B, N), -1, dtype=np.int32)
    rank = np.zeros((B, N), dtype=np.int32)
    score = np.zeros((B, N), dtype=np.float32)
    steps = np.zeros(B, dtype=np.int32)
    for b in range(B):
        heap = [(-float(root_logp[b, r]), -1, r, root_logp[b, r]) for r in range(C)]
        heapq.heapify(heap)
        depth = {-1: 0}
        count = 0
        while count < N:
            if not heap:
                raise DraftError("the candidate heap ran dry before the tree had N nodes")
            new = []
            while heap and len(new) < w and count < N:
                _, p, r, s = heapq.heappop(heap)
                parent[b, count], rank[b, count], score[b, count] = p, r, s
                depth[count] = depth[p] + 1
                new.append(count)
                count += 1
            steps[b] += 1
            for j in new:
                if depth[j] >= max_depth:
                    continue
                for r in range(C):
                    s = np.float32(score[b, j] + node_logp[b, j, r])
                    heapq.heappush(heap, (-float(s), j, r, s))
    return parent, rank, score, steps
