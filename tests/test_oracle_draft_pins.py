"""Pins for the host references of the two steps around verification
(oracle/draft.py): the greedy accepted-node walk and top-w best-first tree
construction.  Each check is against something other than the reference
itself: hand-worked examples (golden fixtures), closed forms for special
cases, and brute force over every candidate in tiny cases.
"""
import itertools

import numpy as np
import pytest

import gdn_inputs as G
from oracle import draft as D
from tests.conftest import read_golden


def ints(x):
    return [int(round(v)) for v in x]


# ----------------------------------------------------------------------------
# accepted-node selection
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["a", "b", "c"])
def test_accept_hand_worked(case):
    gold = read_golden("accept_tree7.txt")
    parent = np.array([ints(gold["parent"])])
    acc, n = D.accept_path(parent, np.array([ints(gold["draft_" + case])]),
                           np.array([ints(gold["target_" + case])]))
    assert acc.tolist() == ints(gold["accepted_" + case])
    assert n.tolist() == ints(gold["len_" + case])


def test_accept_chain_closed_form():
    """on a chain, node i is accepted iff every drafted token up to i equals
    the verifier's choice before it: the accepted length is the first
    mismatch position"""
    rng = np.random.default_rng(3)
    N = 40
    parent = G.tree_chain(1, N)
    for trial in range(50):
        target = rng.integers(0, 5, size=(1, N + 1))
        draft = target[:, :N].copy()
        m = int(rng.integers(0, N + 1))
        if m < N:
            draft[0, m] = target[0, m] + 1
        acc, n = D.accept_path(parent, draft, target)
        assert n[0] == m and acc[0] == m - 1


def _deepest_matching(parent_row, draft_row, target_row):
    """brute force: the deepest node whose whole root path matches (each node
    s on it drafts the verifier's choice after its parent)"""
    best, best_depth = -1, 0
    for i in range(len(parent_row)):
        s, ok, d = i, True, 0
        while s >= 0:
            ok &= draft_row[s] == target_row[parent_row[s] + 1]
            s, d = parent_row[s], d + 1
        if ok and d > best_depth:
            best, best_depth = i, d
    return best, best_depth


@pytest.mark.parametrize("seed", range(6))
def test_accept_brute_force_distinct_siblings(seed):
    """with distinct sibling tokens the matching path is unique, so the greedy
    walk ends at the deepest node whose whole path matches"""
    rng = G.rng_for(seed, 40)
    parent = G.tree_best_first(rng, 8, 60, 10)
    draft, target = G.make_draft_tokens(parent, rng, vocab=50, p_match=0.85)
    acc, n = D.accept_path(parent, draft, target)
    for b in range(8):
        assert (acc[b], n[b]) == _deepest_matching(parent[b], draft[b], target[b])


def test_accept_rejects_invalid_tree():
    with pytest.raises(D.DraftError):
        D.accept_path(np.array([[-1, 2, 0]]), np.zeros((1, 3), int), np.zeros((1, 4), int))


# ----------------------------------------------------------------------------
# top-w best-first construction
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("w", [1, 2])
def test_build_hand_worked(w):
    gold = read_golden("build_tree6.txt")
    root = np.array([gold["root_logp"]], np.float32)
    node = np.array(gold["node_logp"], np.float32).reshape(1, 6, 2)
    parent, rank, score, steps = D.tree_build(root, node, N=6, w=w, max_depth=2)
    assert parent[0].tolist() == ints(gold[f"parent_w{w}"])
    assert rank[0].tolist() == ints(gold[f"rank_w{w}"])
    assert score[0].tolist() == gold[f"score_w{w}"]
    assert steps[0] == ints(gold[f"steps_w{w}"])[0]


def _top_n_of_candidate_tree(root, row, N, max_depth):
    """every node of the candidate tree down to the depth cap, when every
    node's candidates score the same row: node (r1 .. rd) scores
    root[r1] + row[r2] + ... + row[rd], summed in fp32 from the root; the N
    best scores, and a map from rank path to score"""
    C = len(root)
    nodes = []
    for d in range(1, max_depth + 1):
        for path in itertools.product(range(C), repeat=d):
            s = np.float32(root[path[0]])
            for r in path[1:]:
                s = np.float32(s + row[r])
            nodes.append((float(s), path))
    scores = sorted((sc for sc, _ in nodes), reverse=True)
    return scores[:N], {path: sc for sc, path in nodes}


@pytest.mark.parametrize("seed", range(5))
def test_build_w1_is_the_best_n_candidates(seed):
    """one expansion per step: since a child never outscores its parent, the
    tree holds exactly the N best nodes of the candidate tree (brute force)"""
    rng = np.random.default_rng(seed)
    C, N, cap = 3, 14, 4
    root = np.sort(-rng.random(C).astype(np.float32) * 3)[::-1].astype(np.float32)
    row = np.sort(-rng.random(C).astype(np.float32) * 3)[::-1].astype(np.float32)
    node = np.tile(row, (1, N, 1)).astype(np.float32)
    parent, rank, score, steps = D.tree_build(root[None], node, N=N, w=1, max_depth=cap)
    best, score_of = _top_n_of_candidate_tree(root, row, N, cap)
    # every built node is a node of the candidate tree with its score, and
    # the scores are the N best (paths that permute the same ranks may tie)
    paths = set()
    for j in range(N):
        path, s = [], j
        while s >= 0:
            path.append(int(rank[0, s]))
            s = parent[0, s]
        path = tuple(path[::-1])
        assert score_of[path] == float(score[0, j])
        paths.add(path)
    assert len(paths) == N
    assert sorted(map(float, score[0]), reverse=True) == best
    assert steps[0] == N
    assert list(score[0]) == sorted(score[0], reverse=True)


def test_build_one_step_takes_the_best_prefix_candidates():
    """w >= N with at least N candidates: a single step, every node a child of
    the prefix, in rank order"""
    rng = np.random.default_rng(1)
    C, N = 12, 9
    root = np.sort(-rng.random((2, C)).astype(np.float32), axis=1)[:, ::-1].copy()
    node = np.sort(-rng.random((2, N, C)).astype(np.float32), axis=2)[:, :, ::-1].copy()
    parent, rank, score, steps = D.tree_build(root, node, N=N, w=N, max_depth=5)
    assert (parent == -1).all() and (rank == np.arange(N)).all() and (steps == 1).all()
    assert np.array_equal(score, root[:, :N])


def test_build_steps_when_the_prefix_candidates_dominate():
    """prefix candidates all better than anything deeper: the first
    ceil(N / w) steps take prefix candidates w at a time"""
    C, N, w = 32, 30, 7
    root = -np.arange(C, dtype=np.float32) * 1e-3
    node = np.full((1, N, C), -10.0, np.float32)
    parent, rank, score, steps = D.tree_build(root[None], node, N=N, w=w, max_depth=3)
    assert steps[0] == -(-N // w) and (parent == -1).all()


@pytest.mark.parametrize("cap", [1, 2, 3])
def test_build_depth_cap_and_invariants(cap):
    rng = G.rng_for(7)
    N = 40 if cap > 1 else 8   # a depth-1 tree holds at most the 8 prefix candidates
    root, node = G.make_candidate_logp(rng, 3, N, 8)
    parent, rank, score, steps = D.tree_build(root, node, N=N, w=3, max_depth=cap)
    for b in range(3):
        depth = {}
        for j, p in enumerate(parent[b]):
            assert p < j
            depth[j] = 1 if p < 0 else depth[p] + 1
            assert depth[j] <= cap
            base = root[b, rank[b, j]] if p < 0 else np.float32(score[b, p] + node[b, p, rank[b, j]])
            assert score[b, j] == base


def test_build_rejects_unsorted_rows_and_a_dry_heap():
    root = np.array([[-1.0, -0.5]], np.float32)
    with pytest.raises(D.DraftError):
        D.tree_build(root, np.zeros((1, 4, 2), np.float32), N=4, w=1, max_depth=3)
    with pytest.raises(D.DraftError):   # one candidate per node, depth cap 2: only 2 nodes possible
        D.tree_build(np.array([[-1.0]], np.float32), np.full((1, 3, 1), -1.0, np.float32), N=3, w=1, max_depth=2)
