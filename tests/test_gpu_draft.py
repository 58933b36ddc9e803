"""GPU parity of the steps around verification: top-w best-first tree
construction (gdn_tree_build) and greedy accepted-node selection
(gdn_accept_path), called through the C ABI and compared bit for bit with
the host references of oracle/draft.py on seeded synthetic inputs; and the
device chain verify -> accept -> commit against the fp64 oracle."""
import sys

import numpy as np
import pytest

import gdn_inputs as G
import oracle
from oracle import draft as D

torch = pytest.importorskip("torch")
gdn = pytest.importorskip("gated_deltanet_tree_gdn_amd")

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    gdn.load_library()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# ----------------------------------------------------------------------------
# accepted-node selection
# ----------------------------------------------------------------------------

def check_accept(parent, draft, target, what):
    want_acc, want_len = D.accept_path(parent, draft, target)
    acc, n, status = gdn.gdn_accept_path(dev(parent), dev(draft), dev(target))
    torch.cuda.synchronize()
    say(f"  {what}: mean accepted length {want_len.mean():.2f}")
    assert np.array_equal(acc.cpu().numpy(), want_acc), what
    assert np.array_equal(n.cpu().numpy(), want_len), what
    assert not status.cpu().numpy().any()


@pytest.mark.parametrize("N,depth,p", [(128, 16, 0.8), (256, 24, 0.9), (64, 16, 0.5), (200, 40, 1.0)])
def test_accept_best_first(N, depth, p):
    rng = G.rng_for(N, 500)
    parent = G.tree_best_first(rng, 32, N, depth)
    draft, target = G.make_draft_tokens(parent, rng, p_match=p)
    say(f"[accept] best-first B=32 N={N} p_match={p}")
    check_accept(parent, draft, target, f"best-first N={N}")


def test_accept_edge_cases():
    rng = G.rng_for(3, 501)
    say("[accept] chains, ties, forests, single nodes")
    # full-length chain match, and a chain that stops at every position
    N = 256
    parent = G.tree_chain(8, N)
    target = rng.integers(0, 100, size=(8, N + 1)).astype(np.int32)
    draft = target[:, :N].copy()
    for b, m in enumerate([N, 0, 1, 63, 64, 128, 200, 255]):
        if m < N:
            draft[b, m] += 1
    check_accept(parent, draft, target, "chains")
    # siblings with equal tokens (ties go to the lower index) and forests
    parent = G.tree_uniform(rng, 16, 40)
    parent[rng.random((16, 40)) < 0.15] = -1
    draft = rng.integers(0, 3, size=(16, 40)).astype(np.int32)
    target = rng.integers(0, 3, size=(16, 41)).astype(np.int32)
    check_accept(parent, draft, target, "ties and forests")
    check_accept(np.full((4, 1), -1, np.int32), np.arange(4, dtype=np.int32)[:, None],
                 np.array([[0, 5], [9, 9], [2, 0], [3, 3]], np.int32), "single nodes")


def test_accept_invalid_tree_flagged():
    parent = np.array([[-1, 0, 5, 1], [-1, 0, 1, 2]], np.int32)
    acc, n, status = gdn.gdn_accept_path(dev(parent), dev(np.zeros((2, 4), np.int32)),
                                         dev(np.zeros((2, 5), np.int32)))
    assert status.cpu().tolist() == [6, 0]
    assert acc.cpu().tolist()[1] == 3


def test_verify_accept_commit_on_device():
    """the accepted node goes from gdn_accept_path to gdn_commit_path without
    leaving the device; S_new matches the oracle's commit of the host
    reference's accepted node"""
    cfg = G.CONFIGS["bestfirst_b32n128"]
    inp = G.make_inputs(cfg, seed=8)
    rng = G.rng_for(8, 502)
    draft, target = G.make_draft_tokens(inp["parent"], rng)
    d = G.to_device(inp)
    say("[accept] verify -> accept -> commit at B=32 N=128")
    o, ctx = gdn.verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"])
    acc, n, status = gdn.gdn_accept_path(d["parent"], dev(draft), dev(target))
    S_new = gdn.gdn_commit_path(ctx, acc)
    gdn.gdn_ctx_status(ctx)
    want_acc, _ = D.accept_path(inp["parent"], draft, target)
    assert np.array_equal(acc.cpu().numpy(), want_acc)
    want = oracle.commit_inputs(inp, accepted=want_acc)
    got = S_new.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= 1e-3 and np.abs(got - want).max() <= 5e-3


# ----------------------------------------------------------------------------
# tree construction
# ----------------------------------------------------------------------------

def check_build(root, node, w, cap, what):
    N = node.shape[1]
    want = D.tree_build(root, node, N=N, w=w, max_depth=cap)
    got = gdn.gdn_tree_build(dev(root), dev(node), w, cap)
    torch.cuda.synchronize()
    names = ("parent", "cand_rank", "score", "steps")
    for name, x, y in zip(names, got, want):
        assert np.array_equal(x.cpu().numpy(), y), f"{what}: {name} differs"
    assert not got[4].cpu().numpy().any()
    say(f"  {what}: steps {int(want[3].max())}, max depth {G.tree_stats(want[0])['max_depth']}")


# N = 64, 128, 200, 256: two to five positions per lane in the kernel
@pytest.mark.parametrize("N,cap", [(128, 16), (256, 24), (64, 16), (200, 24)])
@pytest.mark.parametrize("w", [1, 4, 16, 64])
def test_build_matches_reference(N, cap, w):
    rng = G.rng_for(N + w, 510)
    root, node = G.make_candidate_logp(rng, 32, N, 8)
    say(f"[build] B=32 N={N} w={w} cap={cap}")
    check_build(root, node, w, cap, f"N={N} w={w}")


@pytest.mark.parametrize("N", [63, 127, 191, 254])
def test_build_full_lanes(N):
    # the largest N for one to four positions per lane (the prefix is a
    # position too): every lane's last head slot holds a position
    rng = G.rng_for(N, 512)
    root, node = G.make_candidate_logp(rng, 32, N, 8)
    say(f"[build] B=32 N={N} w=4 cap=24")
    check_build(root, node, 4, 24, f"N={N} w=4")


def test_build_edge_cases():
    rng = G.rng_for(1, 511)
    say("[build] edge cases")
    # one candidate per node: a chain
    root, node = G.make_candidate_logp(rng, 4, 50, 1)
    check_build(root, node, 3, 60, "one candidate (chain)")
    # 32 candidates, depth cap 1: every node a child of the prefix
    root, node = G.make_candidate_logp(rng, 4, 32, 32)
    check_build(root, node, 5, 1, "depth cap 1")
    # ties everywhere: equal dyadic scores
    root = np.full((3, 4), -1.0, np.float32)
    node = np.full((3, 30, 4), -0.5, np.float32)
    check_build(root, node, 3, 6, "equal scores")
    # w larger than N, N = 1, N = 256 with w = 256
    root, node = G.make_candidate_logp(rng, 2, 1, 8)
    check_build(root, node, 9, 4, "N = 1")
    root, node = G.make_candidate_logp(rng, 2, 256, 32)
    check_build(root, node, 256, 24, "w = N = 256")


def test_build_flags_unsorted_rows_and_a_dry_heap():
    root = np.array([[-1.0, -2.0], [-1.0, -2.0]], np.float32)
    node = np.full((2, 4, 2), -1.0, np.float32)
    node[0, 2] = [-3.0, -1.0]          # not best first
    got = gdn.gdn_tree_build(dev(root), dev(node), 1, 8)
    assert got[4].cpu().tolist() == [2, 0]
    root1 = np.full((1, 1), -1.0, np.float32)     # one candidate, depth cap 2: two nodes at most
    got = gdn.gdn_tree_build(dev(root1), dev(np.full((1, 3, 1), -1.0, np.float32)), 1, 2)
    assert got[4].cpu().tolist() == [6]


def test_build_then_verify():
    """a tree built on the device feeds gdn_tree_verify directly"""
    cfg = G.CONFIGS["bestfirst_b32n128"]
    rng = G.rng_for(2, 512)
    root, node = G.make_candidate_logp(rng, cfg.B, cfg.N, 8)
    parent, _, _, _, status = gdn.gdn_tree_build(dev(root), dev(node), 8, 16)
    inp = G.make_inputs(cfg, seed=9, parent=parent.cpu().numpy())
    d = G.to_device(inp)
    d["parent"] = parent
    say("[build] build -> verify at B=32 N=128")
    o, ctx = gdn.verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"])
    gdn.gdn_ctx_status(ctx)
    want = oracle.verify_inputs(inp)
    got = o.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= 1e-3 and np.abs(got - want).max() <= 5e-3
