"""GPU parity of the delayed commit fused into the next verify
(gdn_commit_verify, called through the C ABI) against the fp64 oracle run as
its two steps: the commit of the recorded tree at the accepted node, then
the verify of the new tree on the committed state.

Bars as for every whole output tensor here: rel-L2 <= 1e-3 and max-abs <=
5e-3 against the oracle, for S_next and for o.  Cases cover one-chunk and
multi-chunk accepted paths (path longer than 16 nodes), new trees deep
enough for the per-node walk, N <= 64 and ragged N, d_k = d_v = 64, empty
and out-of-range accepted nodes, the in-place form, a chain of three
decoding steps, the full B = 32, N = 128 workload, and fp32 q/k/v (which
runs the two steps as separate launches).
"""
import sys

import numpy as np
import pytest

import gdn_inputs as G
import oracle

torch = pytest.importorskip("torch")
gdn = pytest.importorskip("gated_deltanet_tree_gdn_amd")

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS = 5e-3
BASE = G.CONFIGS["bestfirst_b32n128"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    gdn.load_library()


def assert_close(x, y, what):
    x = np.asarray(x, dtype=np.float64)
    rel = np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)
    mab = float(np.abs(x - y).max()) if x.size else 0.0
    say(f"  {what}: rel-L2 {rel:.3e}  max-abs {mab:.3e}")
    assert rel <= REL_L2 and mab <= MAX_ABS, f"{what}: rel-L2 {rel:.3e} max-abs {mab:.3e}"


def inputs(cfg, seed, tree=None):
    c = G.shrink(cfg, tree=tree) if tree else cfg
    inp = G.make_inputs(c, seed=seed)
    return inp, G.to_device(inp)


def deepest(parent):
    """the deepest node of each tree (lowest index among equals)"""
    B, N = parent.shape
    out = np.empty(B, np.int32)
    for b in range(B):
        d = np.zeros(N, int)
        for i in range(N):
            d[i] = 1 if parent[b, i] < 0 else d[parent[b, i]] + 1
        out[b] = int(np.argmax(d))
    return out


def run_step(ctx, inp0, inp1, d1, accepted, read_as=None):
    """one fused step on the device and the oracle's two steps (the oracle
    commits at `read_as`, default the accepted nodes themselves)"""
    acc = torch.from_numpy(np.ascontiguousarray(accepted, dtype=np.int32)).cuda()
    o, S = gdn.gdn_commit_verify(ctx, acc, d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], d1["parent"])
    torch.cuda.synchronize()
    S_ref = oracle.commit_inputs(inp0, accepted=accepted if read_as is None else read_as)
    o_ref = oracle.verify_inputs(dict(inp1, S0=S_ref))
    return o, S, o_ref, S_ref


@pytest.mark.parametrize("prev_tree,new_tree,N,dk,dv", [
    ("best_first", "best_first", 128, 128, 128),   # one-chunk path, MFMA verify
    ("chain", "best_first", 128, 128, 128),        # up to 8 chunks
    ("best_first", "chain", 128, 128, 128),        # new tree walked per node
    ("chain", "chain", 77, 128, 128),              # both, ragged N
    ("best_first", "best_first", 64, 128, 128),    # N <= 64 kernels
    ("chain", "best_first", 45, 64, 64),           # d_k = d_v = 64, ragged
    ("best_first", "uniform", 100, 64, 128),
])
def test_commit_verify_matches_oracle(prev_tree, new_tree, N, dk, dv):
    cfg = G.shrink(BASE, B=4, N=N, d_k=dk, d_v=dv)
    inp0, d0 = inputs(cfg, 300 + N, prev_tree)
    inp1, d1 = inputs(cfg, 301 + N, new_tree)
    rng = G.rng_for(N, 310)
    # the deepest node, a random node, the root alone, and no node
    acc = np.array([deepest(inp0["parent"])[0], rng.integers(0, N), 0, -1], np.int32)
    say(f"[commit-verify] prev {prev_tree} new {new_tree} N={N} d_k={dk} d_v={dv} accepted {acc.tolist()}")
    _, ctx = gdn.verify(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["parent"], d0["S0"])
    o, S, o_ref, S_ref = run_step(ctx, inp0, inp1, d1, acc)
    gdn.gdn_ctx_status(ctx)
    assert_close(S.cpu().numpy(), S_ref, "S_next")
    assert_close(o.cpu().numpy(), o_ref, "o")


def test_commit_verify_out_of_range_accepted():
    """an accepted node outside [-1, N-1] is reported and read as -1: that
    sequence keeps S0 exactly and the others are unaffected"""
    cfg = G.shrink(BASE, B=4)
    inp0, d0 = inputs(cfg, 320)
    inp1, d1 = inputs(cfg, 321)
    acc = np.array([cfg.N, 5, -7, 60], np.int32)
    say("[commit-verify] out-of-range accepted nodes")
    _, ctx = gdn.verify(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["parent"], d0["S0"])
    read_as = np.where((acc < -1) | (acc >= cfg.N), -1, acc).astype(np.int32)
    o, S, o_ref, S_ref = run_step(ctx, inp0, inp1, d1, acc, read_as)
    with pytest.raises(gdn.GdnError, match="accepted"):
        gdn.gdn_ctx_status(ctx)
    got = S.cpu().numpy()
    assert np.array_equal(got[0], inp0["S0"][0]) and np.array_equal(got[2], inp0["S0"][2])
    assert_close(got, S_ref, "S_next")
    assert_close(o.cpu().numpy(), o_ref, "o")


def test_commit_verify_in_place_and_chained():
    """three decoding steps, the state updated in place: verify, then two
    fused steps, each against the oracle's chain"""
    cfg = G.shrink(BASE, B=6)
    steps = [inputs(cfg, 330 + s, "chain" if s == 1 else None) for s in range(3)]
    rng = G.rng_for(6, 331)
    say("[commit-verify] three steps in place")
    inp0, d0 = steps[0]
    state = d0["S0"].clone()
    _, ctx = gdn.verify(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["parent"], state)
    S_ref = inp0["S0"].astype(np.float64)
    prev = inp0
    for s in (1, 2):
        inp, d = steps[s]
        acc = rng.integers(-1, cfg.N, size=cfg.B).astype(np.int32)
        acc[0] = deepest(prev["parent"])[0]
        o, S = gdn.gdn_commit_verify(ctx, torch.from_numpy(acc).cuda(), d["q"], d["k"], d["v"], d["g"],
                                     d["beta"], d["parent"], S_next=state)
        assert S.data_ptr() == state.data_ptr()
        gdn.gdn_ctx_status(ctx)
        S_ref = oracle.commit_inputs(dict(prev, S0=S_ref), accepted=acc)
        o_ref = oracle.verify_inputs(dict(inp, S0=S_ref))
        assert_close(state.cpu().numpy(), S_ref, f"S after step {s}")
        assert_close(o.cpu().numpy(), o_ref, f"o of step {s}")
        prev = inp
    # the record now holds the last tree with S0 = state: a plain commit
    # after the chain continues it
    acc = deepest(prev["parent"])
    S_last = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
    gdn.gdn_ctx_status(ctx)
    assert_close(S_last.cpu().numpy(), oracle.commit_inputs(dict(prev, S0=S_ref), accepted=acc), "final commit")


def test_commit_verify_full_workload():
    """the B = 32, N = 128 best-first workload, every output"""
    inp0, d0 = inputs(BASE, 340)
    inp1, d1 = inputs(BASE, 341)
    rng = G.rng_for(32, 342)
    acc = np.where(rng.random(BASE.B) < 0.1, -1, deepest(inp0["parent"])).astype(np.int32)
    say(f"[commit-verify] B=32 N=128 full, {int((acc < 0).sum())} sequences with no accepted node")
    _, ctx = gdn.verify(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["parent"], d0["S0"])
    o, S, o_ref, S_ref = run_step(ctx, inp0, inp1, d1, acc)
    gdn.gdn_ctx_status(ctx)
    assert_close(S.cpu().numpy(), S_ref, "S_next")
    assert_close(o.cpu().numpy(), o_ref, "o")


def test_commit_verify_fp32_two_launches():
    cfg = G.shrink(G.CONFIGS["tiny_f32"], B=3, N=40, H_k=2, H_v=4)
    inp0, d0 = inputs(cfg, 350)
    inp1, d1 = inputs(cfg, 351)
    acc = np.array([39, -1, 7], np.int32)
    say("[commit-verify] fp32 q/k/v")
    _, ctx = gdn.verify(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["parent"], d0["S0"])
    o, S, o_ref, S_ref = run_step(ctx, inp0, inp1, d1, acc)
    gdn.gdn_ctx_status(ctx)
    assert_close(S.cpu().numpy(), S_ref, "S_next")
    assert_close(o.cpu().numpy(), o_ref, "o")


def test_commit_verify_needs_a_recorded_verify():
    cfg = G.shrink(BASE, B=2, N=16)
    inp1, d1 = inputs(cfg, 360)
    ctx = gdn.GdnContext(cfg.B, cfg.N, cfg.H_k, cfg.H_v, cfg.d_k, cfg.d_v)
    acc = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    with pytest.raises(gdn.GdnError, match="STATE|verify"):
        gdn.gdn_commit_verify(ctx, acc, d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], d1["parent"])
