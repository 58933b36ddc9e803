"""GPU parity: the HIP library (called through its C ABI) against the fp64
oracle, element by element, on seeded inputs; plus the exactness and
invariance properties of rollback-free tree verification.

Bars (stated here, applied to every whole output tensor, o and S_new):
  rel-L2 = ||x - y||_2 / ||y||_2 <= 1e-3   and   max |x - y| <= 5e-3,
with y the fp64 oracle, on bf16 q/k/v and an fp32 state.  Ancestor sets,
depths and the hand-worked dyadic example must match bit for bit.
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    gdn.load_library()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def errors(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    rel = np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)
    mab = float(np.max(np.abs(x - y))) if x.size else 0.0
    return rel, mab


def assert_close(x, y, what):
    rel, mab = errors(x, y)
    say(f"  {what}: rel-L2 {rel:.3e}  max-abs {mab:.3e}")
    assert rel <= REL_L2 and mab <= MAX_ABS, f"{what}: rel-L2 {rel:.3e} max-abs {mab:.3e}"


def run_verify(d, ctx=None):
    o, ctx = gdn.verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"], ctx=ctx)
    return o, ctx


def case_inputs(name, **shrink):
    cfg = G.CONFIGS[name]
    if shrink:
        cfg = G.shrink(cfg, **shrink)
    inp = G.make_inputs(cfg, seed=0)
    return cfg, inp, G.to_device(inp)


# ----------------------------------------------------------------------------
# parity on the workloads
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "chain64", "bestfirst128", "batched_commit", "bestfirst_b32n128"])
def test_parity_workload(name):
    cfg, inp, d = case_inputs(name)
    say(f"[parity] {name}: B={cfg.B} N={cfg.N} Hk={cfg.H_k} Hv={cfg.H_v} d={cfg.d_k} {cfg.dtype}")
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    want = oracle.verify_inputs(inp)
    assert_close(o.cpu().numpy(), want, f"{name} o")
    acc = inp.get("accepted")
    if acc is None:
        acc = G.rng_for(1).integers(-1, cfg.N, size=cfg.B).astype(np.int32)
    S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
    gdn.gdn_ctx_status(ctx)
    assert_close(S_new.cpu().numpy(), oracle.commit_inputs(inp, accepted=acc), f"{name} S_new")


def host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def layer_to_host(d):
    """every tensor of one device layer as fp64 host arrays (parent int32)"""
    out = {n: host64(d[n]) for n in ("q", "k", "v", "g", "beta", "S0")}
    out["parent"] = d["parent"].cpu().numpy()
    return out


def units_to_host(d, units):
    """the (sequence b, value head h) units of one device layer as a batch of
    single-head sequences (H_k = H_v = 1), fp64 host arrays"""
    Hk, Hv = d["q"].shape[2], d["v"].shape[2]
    bs = torch.tensor([b for b, _ in units], device=d["q"].device)
    hs = torch.tensor([h for _, h in units], device=d["q"].device)
    khs = hs // (Hv // Hk)
    return {"q": host64(d["q"][bs, :, khs].unsqueeze(2)), "k": host64(d["k"][bs, :, khs].unsqueeze(2)),
            "v": host64(d["v"][bs, :, hs].unsqueeze(2)), "g": host64(d["g"][bs, :, hs].unsqueeze(2)),
            "beta": host64(d["beta"][bs, :, hs].unsqueeze(2)), "S0": host64(d["S0"][bs, hs].unsqueeze(1)),
            "parent": d["parent"][bs].cpu().numpy()}


STRESS_UNITS_PER_LAYER = 22   # x 47 layers = 1034 sampled units beyond layer 0
STRESS_COMMIT_UNITS = 64


def test_parity_stress48_sampled():
    """48 layers of B=64, N=256, 32 value / 16 key heads, best-first trees of
    depth <= 24 shared by all layers, every layer verified on the GPU.
    Checked against the oracle: all 2048 (b, h) units of layer 0 (o and the
    commit's S_new), and a seeded sample of 22 units in each of layers
    1..47 (1034 units), plus S_new on 64 seeded units of the last layer."""
    cfg = G.CONFIGS["stress48"]
    parent = G.make_tree(cfg, G.rng_for(0, 0))
    rng = G.rng_for(2)
    ctx = None
    checked = 0
    for layer in range(cfg.layers):
        d = G.make_inputs_device(cfg, seed=0, layer=layer, parent=parent)
        if ctx is None:
            ctx = gdn.GdnContext.for_tensors(d["q"], d["v"], d["parent"])
        o, _ = run_verify(d, ctx=ctx)
        gdn.gdn_ctx_status(ctx)
        if layer == 0:
            say(f"[parity] stress48 layer 0: all {cfg.B * cfg.H_v} units")
            host = layer_to_host(d)
            assert_close(o.cpu().numpy(), oracle.verify_inputs(host), "stress48 layer 0 o (every unit)")
            acc = rng.integers(-1, cfg.N, size=cfg.B).astype(np.int32)
            S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
            gdn.gdn_ctx_status(ctx)
            assert_close(S_new.cpu().numpy(), oracle.commit_inputs(host, accepted=acc),
                         "stress48 layer 0 S_new (every unit)")
            checked += cfg.B * cfg.H_v
            del host, S_new
        else:
            units = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.H_v))) for _ in range(STRESS_UNITS_PER_LAYER)]
            say(f"[parity] stress48 layer {layer}: {len(units)} sampled units")
            got = torch.stack([o[b, :, h] for b, h in units]).unsqueeze(2).cpu().numpy()
            want = oracle.verify_inputs(units_to_host(d, units))
            assert_close(got, want, f"stress48 layer {layer} sampled o")
            checked += len(units)
        if layer == cfg.layers - 1:
            units = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.H_v))) for _ in range(STRESS_COMMIT_UNITS)]
            acc = rng.integers(-1, cfg.N, size=cfg.B).astype(np.int32)
            S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
            gdn.gdn_ctx_status(ctx)
            gotS = torch.stack([S_new[b, h] for b, h in units]).unsqueeze(1).cpu().numpy()
            wantS = oracle.commit_inputs(units_to_host(d, units), accepted=np.array([acc[b] for b, _ in units]))
            say(f"[parity] stress48 layer {layer}: S_new on {len(units)} sampled units")
            assert_close(gotS, wantS, f"stress48 layer {layer} sampled S_new")
        del d, o
    say(f"[parity] stress48: {checked} (layer, b, h) units checked")
    assert checked >= cfg.B * cfg.H_v + 1024


# ----------------------------------------------------------------------------
# exact results
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("which", ["tree", "chain"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_dyadic_example_bit_exact(which, dtype, d):
    from tests.conftest import read_golden
    gold = read_golden("dyadic_tree3.txt")
    say(f"[exact] dyadic {which} {dtype} d={d}")
    N = 3
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    e0 = torch.zeros(d)
    e0[0] = 1
    q = e0.repeat(1, N, 1, 1).to(tdt).cuda().contiguous()
    k = q.clone()
    v = torch.zeros(1, N, 1, d)
    v[0, :, 0, 0] = torch.tensor(gold["v"])
    v = v.to(tdt).cuda().contiguous()
    g = torch.full((1, N, 1), gold["g"][0]).cuda()
    beta = torch.full((1, N, 1), gold["beta"][0]).cuda()
    S0 = torch.zeros(1, 1, d, d)
    S0[0, 0, 0, 0] = gold["S0"][0]
    S0 = S0.cuda()
    parent = torch.tensor([gold["parent_" + which]], dtype=torch.int32).cuda()
    o, ctx = gdn.verify(q, k, v, g, beta, parent, S0)
    want = torch.zeros(1, N, 1, d)
    want[0, :, 0, 0] = torch.tensor(gold["o_" + which])
    assert torch.equal(o.cpu(), want)
    for a in range(N):
        Sn = gdn.gdn_commit_path(ctx, torch.tensor([a], dtype=torch.int32).cuda())
        wantS = torch.zeros(1, 1, d, d)
        wantS[0, 0, 0, 0] = gold["commit_" + which][a]
        assert torch.equal(Sn.cpu(), wantS)


@pytest.mark.parametrize("N", [1, 5, 31, 32, 33, 100, 256])
def test_ancestors_bit_exact(N):
    rng = G.rng_for(N)
    trees = [G.tree_uniform(rng, 2, N), G.tree_chain(1, N), G.tree_best_first(rng, 2, N, 24 if N > 100 else 8)]
    forest = G.tree_uniform(rng, 1, N)
    forest[0, rng.random(N) < 0.2] = -1
    trees.append(forest)
    parent = np.concatenate(trees).astype(np.int32)
    say(f"[exact] ancestors B={parent.shape[0]} N={N}")
    anc, depth, status = gdn.gdn_tree_ancestors(torch.from_numpy(parent).cuda())
    want_anc, want_depth = oracle.ancestors(parent)
    assert np.array_equal(anc.cpu().numpy().view(np.uint32), want_anc)
    assert np.array_equal(depth.cpu().numpy(), want_depth)
    assert not status.cpu().numpy().any()


# ----------------------------------------------------------------------------
# properties of rollback-free verification
# ----------------------------------------------------------------------------

def _repeat_bitwise(fn, calls=10):
    first = fn().clone()
    for c in range(1, calls):
        again = fn()
        assert torch.equal(first, again), f"call {c} differs from call 0 " \
            f"({int((first != again).sum())} elements)"
    return first


def test_verify_repeatable_and_prefix_state_untouched_b32n128():
    """the persistent pipelined verify at B=32, N=128 (several (b, h) items
    per workgroup, the tree and dense wavefronts handing over through LDS):
    10 calls bitwise identical; S0 never written"""
    cfg, inp, d = case_inputs("bestfirst_b32n128")
    say("[repeat] verify B=32 N=128, 10 calls")
    S0_before = d["S0"].clone()
    ctx = gdn.GdnContext.for_tensors(d["q"], d["v"], d["parent"])
    o = torch.empty((cfg.B, cfg.N, cfg.H_v, cfg.d_v), dtype=torch.float32, device="cuda:0")

    def call():
        gdn.gdn_tree_verify(ctx, d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"], o=o)
        gdn.gdn_ctx_status(ctx)
        return o

    _repeat_bitwise(call)
    assert torch.equal(d["S0"], S0_before)


def test_verify_repeatable_stress_layer():
    """one layer of the 256-node stress workload: 10 calls bitwise identical"""
    cfg = G.CONFIGS["stress48"]
    parent = G.make_tree(cfg, G.rng_for(0, 0))
    d = G.make_inputs_device(cfg, seed=0, layer=7, parent=parent)
    say("[repeat] verify stress layer B=64 N=256, 10 calls")
    ctx = gdn.GdnContext.for_tensors(d["q"], d["v"], d["parent"])
    o = torch.empty((cfg.B, cfg.N, cfg.H_v, cfg.d_v), dtype=torch.float32, device="cuda:0")

    def call():
        gdn.gdn_tree_verify(ctx, d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"], o=o)
        gdn.gdn_ctx_status(ctx)
        return o

    _repeat_bitwise(call)


def test_commit_repeatable_b32n128():
    """the commit at B=32, N=128: 10 calls bitwise identical"""
    cfg, inp, d = case_inputs("bestfirst_b32n128")
    acc = torch.from_numpy(G.rng_for(0, 77).integers(-1, cfg.N, size=cfg.B).astype(np.int32)).cuda()
    _, ctx = run_verify(d)
    S_new = torch.empty_like(d["S0"])
    say("[repeat] commit B=32 N=128, 10 calls")

    def call():
        gdn.gdn_commit_path(ctx, acc, S_new=S_new)
        gdn.gdn_ctx_status(ctx)
        return S_new

    _repeat_bitwise(call)


def test_prefix_state_untouched_and_deterministic():
    cfg, inp, d = case_inputs("bestfirst128")
    say("[prop] S0 untouched, 10 calls bitwise identical")
    S0_before = d["S0"].clone()
    o1, ctx = run_verify(d)
    for _ in range(9):
        o2, _ = run_verify(d, ctx=ctx)
        assert torch.equal(o1, o2)
    assert torch.equal(d["S0"], S0_before)


def test_subtree_locality_bitwise():
    cfg, inp, d = case_inputs("bestfirst128", H_v=4, H_k=2)
    par = inp["parent"][0]
    anc, _ = oracle.ancestors(inp["parent"])
    o1, ctx = run_verify(d)
    for j in (0, 5, 40, 127):
        say(f"[prop] perturb node {j}")
        d2 = {n: t.clone() for n, t in d.items()}
        d2["k"][0, j] = d2["k"][0, j].flip(-1)
        d2["v"][0, j] *= -2
        d2["g"][0, j] -= 0.3
        d2["beta"][0, j] *= 0.5
        o2, _ = run_verify(d2)
        desc = np.array([(anc[0, i, j // 32] >> (j % 32)) & 1 for i in range(cfg.N)], bool)
        same = (o1 == o2).reshape(cfg.N, -1).all(dim=1).cpu().numpy()
        assert np.array_equal(same, ~desc)


def test_commit_in_place_and_off_path_invariance():
    cfg, inp, d = case_inputs("batched_commit", B=4)
    acc = torch.from_numpy(inp["accepted"][:4]).cuda()
    o, ctx = run_verify(d)
    S_out = gdn.gdn_commit_path(ctx, acc)
    S_copy = d["S0"].clone()
    o2, ctx2 = run_verify(dict(d, S0=S_copy))
    gdn.gdn_commit_path(ctx2, acc, S_new=S_copy)  # in place
    say("[prop] in-place commit")
    assert torch.equal(S_copy, S_out)
    # nodes off every accepted path: perturb them, the commit is unchanged
    anc, _ = oracle.ancestors(inp["parent"][:4])
    d3 = {n: t.clone() for n, t in d.items()}
    for b in range(4):
        a = int(inp["accepted"][b])
        for j in range(cfg.N):
            if not (anc[b, a, j // 32] >> (j % 32)) & 1:
                d3["v"][b, j] += 1.0
                d3["k"][b, j] = d3["k"][b, j].flip(-1)
                d3["g"][b, j] -= 0.5
    o3, ctx3 = run_verify(d3)
    assert torch.equal(gdn.gdn_commit_path(ctx3, acc), S_out)


def test_relabelled_tree_permutes_outputs():
    cfg, inp, d = case_inputs("bestfirst128", H_v=4, H_k=2)
    par = inp["parent"][0]
    rng = G.rng_for(9)
    placed, order = set(), []
    while len(order) < cfg.N:
        ready = [i for i in range(cfg.N) if i not in placed and (par[i] < 0 or par[i] in placed)]
        pick = ready[rng.integers(len(ready))]
        order.append(pick)
        placed.add(pick)
    new_of = {old: new for new, old in enumerate(order)}
    perm = torch.tensor(order).cuda()
    d2 = {n: d[n][:, perm].contiguous() for n in ("q", "k", "v", "g", "beta")}
    d2["S0"] = d["S0"]
    d2["parent"] = torch.tensor([[new_of[par[o]] if par[o] >= 0 else -1 for o in order]], dtype=torch.int32).cuda()
    o1, _ = run_verify(d)
    o2, _ = run_verify(d2)
    say("[prop] relabelled tree")
    assert_close(o2.cpu().numpy(), o1[:, perm].cpu().numpy(), "relabelled o")


# ----------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [
    dict(N=1), dict(N=37), dict(N=100, max_depth=40), dict(N=256, max_depth=24), dict(N=256, tree="chain"),
    dict(d_k=64, d_v=64), dict(d_k=64, d_v=128), dict(d_k=128, d_v=64), dict(H_k=2, H_v=8),
    dict(N=33, tree="uniform"), dict(dtype="f32", N=70),
    dict(N=64, tree="chain"), dict(N=128, tree="chain"), dict(N=200, tree="uniform"),
    dict(N=160, d_k=64, d_v=128), dict(N=256, d_k=128, d_v=64, max_depth=24), dict(N=140, d_k=64, d_v=64),
    dict(N=180, H_k=2, H_v=6, max_depth=24), dict(N=150, H_k=4, H_v=4, max_depth=24),
])
def test_edge_shapes(shape):
    base = G.shrink(G.CONFIGS["bestfirst128"], B=2, H_k=2, H_v=4)
    cfg = G.shrink(base, **shape)
    inp = G.make_inputs(cfg, seed=3)
    say(f"[edge] {shape}")
    d = G.to_device(inp)
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), f"edge {shape} o")
    acc = np.array([cfg.N - 1, -1], np.int32)
    S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
    assert_close(S_new.cpu().numpy(), oracle.commit_inputs(inp, accepted=acc), f"edge {shape} S_new")


def test_forest():
    cfg = G.shrink(G.CONFIGS["bestfirst128"], B=2, H_k=1, H_v=2, N=64)
    inp = G.make_inputs(cfg, seed=4)
    inp["parent"][:, [10, 20, 33]] = -1
    say("[edge] forest")
    d = G.to_device(inp)
    o, ctx = run_verify(d)
    assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), "forest o")


def test_empty_tree_is_noop():
    cfg = G.shrink(G.CONFIGS["bestfirst128"], B=2, H_k=1, H_v=1, N=0)
    inp = G.make_inputs(cfg)
    d = G.to_device(inp)
    o, ctx = run_verify(d)
    assert o.shape == (2, 0, 1, 128)


def test_invalid_tree_and_accepted_are_flagged():
    cfg, inp, d = case_inputs("bestfirst128", B=3, H_k=1, H_v=2, N=40)
    d["parent"][1, 7] = 9   # a forward edge
    d["parent"][2, 3] = -5
    say("[err] invalid tree")
    o, ctx = run_verify(d)
    with pytest.raises(gdn.GdnError) as ei:
        gdn.gdn_ctx_status(ctx)
    assert ei.value.status == "GDN_ERR_TREE"
    cfg, inp, d = case_inputs("bestfirst128", B=3, H_k=1, H_v=2, N=40)
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    say("[err] invalid accepted")
    gdn.gdn_commit_path(ctx, torch.tensor([3, 40, -1], dtype=torch.int32).cuda())
    with pytest.raises(gdn.GdnError) as ei:
        gdn.gdn_ctx_status(ctx)
    assert ei.value.status == "GDN_ERR_ACCEPT"
    _, _, status = gdn.gdn_tree_ancestors(torch.tensor([[-1, 0, 5, 1]], dtype=torch.int32).cuda())
    assert status.cpu().tolist() == [6]


@pytest.mark.parametrize("name", ["chain64", "bestfirst128", "batched_commit"])
def test_walk_kernels_parity(name, monkeypatch):
    """the per-node walk kernels (GDN_FORCE_SIMPLE=1) on bf16 inputs"""
    monkeypatch.setenv("GDN_FORCE_SIMPLE", "1")
    cfg, inp, d = case_inputs(name, B=min(G.CONFIGS[name].B, 4))
    say(f"[walk] {name}")
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), f"walk {name} o")
    acc = np.random.default_rng(5).integers(-1, cfg.N, size=cfg.B).astype(np.int32)
    S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
    gdn.gdn_ctx_status(ctx)
    assert_close(S_new.cpu().numpy(), oracle.commit_inputs(inp, accepted=acc), f"walk {name} S_new")


@pytest.mark.parametrize("tree", ["chain", "best_first"])
def test_commit_every_path_length(tree):
    """commit at every node of one tree: path lengths 1 .. depth, across the
    16-node chunk boundaries of the chunked path update"""
    cfg = G.shrink(G.CONFIGS["bestfirst128"], B=1, H_k=2, H_v=4, N=50, tree=tree, max_depth=50)
    inp = G.make_inputs(cfg, seed=6)
    d = G.to_device(inp)
    say(f"[commit] every node of a {tree} tree")
    _, ctx = run_verify(d)
    for a in range(-1, cfg.N):
        acc = np.array([a], np.int32)
        S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
        assert_close(S_new.cpu().numpy(), oracle.commit_inputs(inp, accepted=acc), f"commit at {a}")


def _mixed_depth_inputs(cfg, seed, chain_every):
    """best-first trees with every `chain_every`-th sequence replaced by a
    chain (whose pair list exceeds what the MFMA kernels keep in LDS for
    N > 55, so those sequences take the per-node walk inside them)"""
    inp = G.make_inputs(cfg, seed=seed)
    par = inp["parent"].copy()
    for b in range(0, cfg.B, chain_every):
        par[b] = np.arange(-1, cfg.N - 1, dtype=np.int32)
    inp["parent"] = par
    return inp


@pytest.mark.parametrize("shape", [
    dict(B=40, N=128, H_k=3, H_v=9),      # 2 heads per workgroup, sequence and key-head changes inside one
    dict(B=24, N=64, H_k=4, H_v=16),      # N <= 64 layout, 2 heads per workgroup
    dict(B=33, N=100, H_k=16, H_v=32),    # 5 heads per workgroup, ragged last workgroup
    dict(B=128, N=128, H_k=16, H_v=32),   # 16 heads per workgroup: the hand-over slots cycle eight times
    dict(B=40, N=77, H_k=3, H_v=9, d_k=64, d_v=64),
    dict(B=40, N=128, H_k=9, H_v=9, d_k=64, d_v=128),
    dict(B=40, N=50, H_k=1, H_v=9, d_k=128, d_v=64),
    dict(B=300, N=1, H_k=1, H_v=2),       # single-node trees, 3 heads per workgroup
    dict(B=64, N=17, H_k=2, H_v=8),       # one node past a 16-node tile
    dict(B=40, N=180, H_k=3, H_v=9),      # trees over 128 nodes, 2 heads per workgroup
    dict(B=30, N=256, H_k=4, H_v=16, d_k=64, d_v=64),
])
def test_pipeline_item_boundaries(shape):
    """several (sequence, head) items per persistent workgroup: sequence,
    key-head and deep-tree (walk) boundaries between consecutive items"""
    cfg = G.shrink(G.CONFIGS["bestfirst_b32n128"], **shape)
    inp = _mixed_depth_inputs(cfg, seed=11, chain_every=7)
    d = G.to_device(inp)
    say(f"[pipeline] {shape}")
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), f"pipeline {shape} o")


def test_workspace_reused_across_trees():
    """trees of more than 128 nodes go through the context's workspace (the
    pair structure, per-sequence deep flags and the values of Z~): three
    verifies on one context, deep and shallow sequences swapping places
    between calls, each against the oracle"""
    cfg = G.shrink(G.CONFIGS["bestfirst_b32n128"], B=4, N=200, H_k=2, H_v=4)
    ctx = None
    for call, chain_every in enumerate((2, 3, 1000)):
        inp = _mixed_depth_inputs(cfg, seed=40 + call, chain_every=chain_every)
        if chain_every == 3:
            # the sequences that were deep in the first call are shallow now
            inp["parent"][[0, 2]] = G.make_inputs(cfg, seed=50)["parent"][[0, 2]]
            inp["parent"][1] = np.arange(-1, cfg.N - 1, dtype=np.int32)
        d = G.to_device(inp)
        say(f"[workspace] call {call + 1}")
        o, ctx = run_verify(d, ctx)
        gdn.gdn_ctx_status(ctx)
        assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), f"workspace call {call + 1} o")


def _spine_tree(N, k, extra):
    """a chain of k nodes, every other node a child of the chain's last
    node, and the last `extra` of those one level deeper (under node k):
    paths that sum to k(k+1)/2 + (N-k)(k+1) + extra nodes"""
    par = np.empty(N, dtype=np.int32)
    par[0] = -1
    par[1:k] = np.arange(0, k - 1)
    par[k:] = k - 1
    par[N - extra:] = k
    return par


@pytest.mark.parametrize("N,spines,expect", [
    (128, {1: (15, 0), 2: (16, 8), 4: (16, 9), 5: (16, 8)}, {1: 1928, 2: 2048, 4: 2049}),
    (256, {0: (23, 0), 3: (24, 44), 4: (24, 45)}, {0: 5868, 3: 6144, 4: 6145}),
])
def test_pair_list_capacity_boundary(N, spines, expect):
    """trees whose paths sum to the most a best-first tree of the pages'
    depth reaches (1928 nodes at N = 128, depth 16; 5868 at N = 256, depth
    24), to the pair-list capacity of the MFMA kernels (2048, 6144) and one
    past it, between best-first trees.  At N = 128 the first two stay on the
    MFMA path and the last takes the per-node walk; at N = 256 the
    two-launch verify solves root paths of up to 24 nodes, so the first
    stays on the MFMA path and the other two (depth 26) are walked"""
    cfg = G.shrink(G.CONFIGS["bestfirst_b32n128"], B=6, N=N, H_k=2, H_v=4)
    inp = G.make_inputs(cfg, seed=5)
    par = inp["parent"].copy()
    for b, (k, extra) in spines.items():
        par[b] = _spine_tree(cfg.N, k, extra)
    totals = [int(t) for t in oracle.ancestors(par)[1].sum(axis=1)]
    assert all(totals[b] == t for b, t in expect.items()), totals
    inp["parent"] = par
    d = G.to_device(inp)
    say(f"[capacity] N={N} path totals {totals}")
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), "capacity boundary o")


def _edge_of_stable_inputs(N, depth, seed):
    """keys at |k|^2 = 2 and beta = 1 (the edge of the stated input range,
    beta in [0, 1] and |k|^2 <= 2), gates -8 along a spine of `depth` nodes
    in sequence 0 (the spine shares one key, so k.k = 2 on every spine pair,
    and the decay across it underflows in fp32), a best-first tree of depth
    <= `depth` in sequence 1"""
    cfg = G.shrink(G.CONFIGS["bestfirst128"], B=2, H_k=2, H_v=4, N=N, max_depth=depth)
    inp = G.make_inputs(cfg, seed=seed)
    rng = np.random.default_rng(seed)
    par = inp["parent"].copy()
    par[0, 0] = -1
    par[0, 1:depth] = np.arange(depth - 1)
    par[0, depth:] = rng.integers(0, depth // 2, size=N - depth)
    inp["parent"] = par
    k = inp["k"] * np.float32(np.sqrt(2.0))
    k[0, :depth] = k[0, :1]
    inp["k_bits"] = G.round_bf16_bits(k)
    inp["k"] = G.bf16_bits_to_f32(inp["k_bits"])
    inp["beta"][:] = 1.0
    inp["g"][0, :depth] = -8.0
    return cfg, inp


@pytest.mark.parametrize("N,depth", [(128, 16), (256, 24)])
def test_solve_at_edge_of_stable_range(N, depth):
    """the row solve of Z~ runs on the Gram values and beta and applies the
    decay afterwards; its intermediates grow by at most 1 + 2 = 3x per path
    node when beta |k_a . k_b| <= 2, finite in fp32 over root paths of 16 and
    24 nodes.  Context verify, commit, the allocation-free verify and
    (N = 128) the fused commit-then-verify, against the oracle"""
    cfg, inp = _edge_of_stable_inputs(N, depth, seed=31)
    d = G.to_device(inp)
    say(f"[edge of stable range] N={N} depth={depth}")
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    o_ref = oracle.verify_inputs(inp)
    assert_close(o.cpu().numpy(), o_ref, "edge-of-stable o")
    o_static = gdn.gdn_tree_verify_static(d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"])
    torch.cuda.synchronize()
    assert_close(o_static.cpu().numpy(), o_ref, "edge-of-stable o (allocation-free)")
    acc = np.array([depth - 1, N - 1], np.int32)
    S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
    assert_close(S_new.cpu().numpy(), oracle.commit_inputs(inp, accepted=acc), "edge-of-stable S_new")
    if N <= 128:
        _, inp2 = _edge_of_stable_inputs(N, depth, seed=32)
        d2 = G.to_device(inp2)
        o2, S2 = gdn.gdn_commit_verify(ctx, torch.from_numpy(acc).cuda(), d2["q"], d2["k"], d2["v"], d2["g"],
                                       d2["beta"], d2["parent"])
        torch.cuda.synchronize()
        S_ref = oracle.commit_inputs(inp, accepted=acc)
        assert_close(S2.cpu().numpy(), S_ref, "edge-of-stable fused S_next")
        assert_close(o2.cpu().numpy(), oracle.verify_inputs(dict(inp2, S0=S_ref)), "edge-of-stable fused o")


def test_tree_runs_span_sequences():
    """the two-launch verify's tree kernel walks runs of consecutive
    (sequence, key head) items, one run per compute unit: with B H_k = 300
    items on 256 compute units a run is two items and every other run
    starts in one sequence and ends in the next; sequence 37 is a chain
    deeper than 24 nodes (walked per node by the dense kernel) between
    ordinary trees"""
    cfg = G.shrink(G.CONFIGS["bestfirst128"], B=100, H_k=3, H_v=6, N=140, max_depth=24, d_k=64, d_v=64)
    inp = G.make_inputs(cfg, seed=41)
    par = inp["parent"].copy()
    par[37] = np.arange(-1, cfg.N - 1, dtype=np.int32)
    inp["parent"] = par
    d = G.to_device(inp)
    say("[runs span sequences] B=100 H_k=3 N=140")
    o, ctx = run_verify(d)
    gdn.gdn_ctx_status(ctx)
    assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), "runs span sequences o")
    acc = np.random.default_rng(41).integers(-1, cfg.N, size=cfg.B).astype(np.int32)
    S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
    assert_close(S_new.cpu().numpy(), oracle.commit_inputs(inp, accepted=acc), "runs span sequences S_new")


def test_side_stream():
    """verify and commit launched on a stream other than the current one
    (default priority), ordered only by that stream"""
    cfg = G.shrink(G.CONFIGS["bestfirst_b32n128"], B=4, H_k=2, H_v=4)
    inp = G.make_inputs(cfg, seed=21)
    d = G.to_device(inp)
    acc_np = np.array([cfg.N - 1, 0, -1, 37], dtype=np.int32)
    acc = torch.from_numpy(acc_np).to("cuda:0")
    ctx = gdn.GdnContext.for_tensors(d["q"], d["v"], d["parent"])
    o = torch.empty((cfg.B, cfg.N, cfg.H_v, cfg.d_v), dtype=torch.float32, device="cuda:0")
    S_new = torch.empty_like(d["S0"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())   # inputs and outputs allocated and filled
    say("[side stream] verify + commit")
    gdn.gdn_tree_verify(ctx, d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"], o=o, stream=side)
    gdn.gdn_commit_path(ctx, acc, S_new=S_new, stream=side)
    gdn.gdn_ctx_status(ctx, stream=side)
    side.synchronize()
    assert_close(o.cpu().numpy(), oracle.verify_inputs(inp), "side-stream o")
    assert_close(S_new.cpu().numpy(), oracle.commit_inputs(inp, accepted=acc_np), "side-stream S_new")
