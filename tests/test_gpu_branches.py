"""GPU parity of the per-branch recurrent baseline (gdn_tree_verify_branches)
against the fp64 oracle, on the workloads the fused verify is checked on; it
is the baseline of the fused/per-branch speed ratio that the bench reports.
Bars as in test_gpu_parity: rel-L2 <= 1e-3 and max-abs <= 5e-3."""
import sys

import numpy as np
import pytest

import gdn_inputs as G
import oracle

torch = pytest.importorskip("torch")
gdn = pytest.importorskip("gated_deltanet_tree_gdn_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    gdn.load_library()


@pytest.mark.parametrize("name,shrink", [("tiny_f32", {}), ("chain64", {}), ("bestfirst128", {}),
                                         ("bestfirst_b32n128", {}), ("bestfirst128", dict(N=256, max_depth=24, B=2)),
                                         ("bestfirst128", dict(d_k=64, d_v=64, B=3, H_k=2, H_v=4, N=90))])
def test_branches_parity(name, shrink):
    cfg = G.CONFIGS[name]
    if shrink:
        cfg = G.shrink(cfg, **shrink)
    inp = G.make_inputs(cfg, seed=4)
    d = G.to_device(inp)
    print(f"[branches] {name} {shrink}", flush=True)
    ctx = gdn.GdnContext.for_tensors(d["q"], d["v"], d["parent"])
    o = gdn.gdn_tree_verify_branches(ctx, d["q"], d["k"], d["v"], d["g"], d["beta"], d["parent"], d["S0"])
    gdn.gdn_ctx_status(ctx)
    want = oracle.verify_inputs(inp)
    got = o.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    mab = np.abs(got - want).max()
    print(f"  rel-L2 {rel:.3e} max-abs {mab:.3e}", flush=True)
    assert rel <= 1e-3 and mab <= 5e-3
    # the context it armed commits like the fused verify's
    acc = np.full(cfg.B, cfg.N - 1, np.int32)
    S_new = gdn.gdn_commit_path(ctx, torch.from_numpy(acc).cuda())
    wantS = oracle.commit_inputs(inp, accepted=acc)
    assert np.linalg.norm(S_new.cpu().numpy() - wantS) / np.linalg.norm(wantS) <= 1e-3
