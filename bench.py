#!/usr/bin/env python3
"""Benchmark: GDN rollback-free tree verification on one MI355X.

The metric is tree-verify throughput: one timed call is gdn_tree_verify
(every node's output in one pass, S0 untouched) on the workload

    best-first proposal trees, depth <= 16, B=32 sequences x N=128 nodes,
    32 value heads sharing 16 key heads, d_k = d_v = 128,
    bf16 q/k/v, fp32 g/beta/S0, fp32 outputs (synthetic, seeded).

Inputs live in HBM before timing starts; R rotating input sets (>= 3x the
256 MB Infinity Cache in total) keep the cache from serving the reads.

Prints ONE JSON line.  `value` is nodes*heads per second of gdn_tree_verify
(B*N*H_v per call over the timed calls).  Beside it: verify followed by
gdn_commit_path (the accepted node's state) as one step, the same step as
the fused gdn_commit_verify (the previous tree's commit inside the next
verify), the roofline of the dominant kernel (verify, measured with HIP
events on the stream it runs on) and the fp64 CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN tree-verify nodes·heads/s per layer at B=32,N=128; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
WORKLOAD = "bestfirst_b32n128"
KERNEL_SOURCES = ["gdn_internal.h", "gdn_mfma.h", "gdn_walk.h", "gdn_fast.hip", "gdn_verify_ws.hip",
                  "gdn_split.hip", "gdn_commit_verify.hip", "gdn_commit.hip"]
STRESS = "stress48"


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_verify_{workload}.json")


def kernel_source_sha() -> str:
    """Hash of the kernel sources' code: line comments and blank lines are
    left out, so that a comment edit keeps the counters taken on the code."""
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_deltanet_tree_gdn_amd", "csrc", s), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def verify_bytes(cfg) -> int:
    """Algorithmic bytes of one verify: read q, k, v, g, beta, parent, S0
    once, write o once (fp32)."""
    B, N, Hk, Hv, dk, dv = cfg.B, cfg.N, cfg.H_k, cfg.H_v, cfg.d_k, cfg.d_v
    e = 2 if cfg.dtype == "bf16" else 4
    return (B * Hv * dv * dk * 4 + B * N * Hv * dv * 4 + B * N * Hv * dv * e
            + 2 * B * N * Hk * dk * e + 2 * B * N * Hv * 4 + B * N * 4)


def verify_flops(cfg, mean_strict_ancestors) -> float:
    """Algorithmic floating-point operations of one verify: per (node, value
    head) 4 d_v d_k for S0 k_i and S0 q_i, plus 2 (d_k + d_v) (2 a + 1) for
    the ancestor dot products and the solve and output updates, with a the
    node's strict-ancestor count (its mean over the trees)."""
    nh = cfg.B * cfg.N * cfg.H_v
    return nh * (4.0 * cfg.d_v * cfg.d_k + 2.0 * (cfg.d_k + cfg.d_v) * (2.0 * mean_strict_ancestors + 1.0))


def commit_bytes(cfg, path_len) -> int:
    """Algorithmic bytes of one commit: read S0 and the accepted path's rows
    (k per key head, v/g/beta per value head), parent and accepted; write
    S_new."""
    B, N, Hk, Hv, dk, dv = cfg.B, cfg.N, cfg.H_k, cfg.H_v, cfg.d_k, cfg.d_v
    e = 2 if cfg.dtype == "bf16" else 4
    rows = int(sum(path_len))
    return (2 * B * Hv * dv * dk * 4 + rows * (Hk * dk * e + Hv * (dv * e + 8)) + B * N * 4 + B * 4)


def commit_verify_bytes(cfg, path_len) -> int:
    """Algorithmic bytes of one fused commit-then-verify: the verify's bytes,
    plus the committed state written once (it is not read back), the
    previous tree's accepted-path rows, parents and accepted nodes."""
    B, N, Hk, Hv, dk, dv = cfg.B, cfg.N, cfg.H_k, cfg.H_v, cfg.d_k, cfg.d_v
    e = 2 if cfg.dtype == "bf16" else 4
    rows = int(sum(path_len))
    return (verify_bytes(cfg) + B * Hv * dv * dk * 4 + rows * (Hk * dk * e + Hv * (dv * e + 8))
            + B * N * 4 + B * 4)


def read_traffic(kernel, workload=WORKLOAD):
    """HBM bytes of one launch of `kernel` ("verify", "commit" or
    "commit_verify") on `workload` from the committed rocprofv3 counters, if
    they were taken on the current kernel sources; else None."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get(kernel, {}).get("hbm_bytes_per_launch")


COPY_CALLS = 5
# kernel-name patterns per role; a verify of more than 128 nodes is the
# tree kernel and then the dense kernel, whose per-launch bytes add up; the
# allocation-free entry point runs the single-launch kernel there
KERNELS = {"verify": ("verify_ws_kernel",), "verify_tree": ("tree_kernel",),
           "verify_dense": ("dense_kernel",), "verify_static": ("verify_fast_kernel",),
           "commit": ("commit_mfma_kernel",), "commit_verify": ("commit_verify_kernel",),
           "copy": ("MulFunctor",)}


def write_traffic(fetch_csv, write_csv, copy_mib, workload):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each kernel, scaled by
    the factor that maps the same counter to the known bytes of the
    calibration copy, written to the workload's traffic file with the kernel
    sources' hash."""
    import csv

    def per_kernel(path, counter):
        vals = {k: [] for k in KERNELS}
        with open(path) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            for k, pats in KERNELS.items():
                if any(pat in r["Kernel_Name"] for pat in pats):
                    vals[k].append(float(r["Counter_Value"]))
        vals["copy"] = vals["copy"][-COPY_CALLS:]
        return {k: (sum(v) / len(v) if v else None) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}

    fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, nw = per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = float(copy_mib << 10)
    ff, fw = copy_kib / fetch["copy"], copy_kib / write["copy"]
    out = {"kernel_source_sha": kernel_source_sha(), "copy_kib": copy_kib,
           "fetch_factor": ff, "write_factor": fw, "dispatches": {"fetch": nf, "write": nw}}
    out["workload"] = workload
    for k in ("verify", "verify_tree", "verify_dense", "verify_static", "commit", "commit_verify"):
        if fetch[k] is None or write[k] is None:
            continue
        out[k] = {"fetch_kib": fetch[k], "write_kib": write[k],
                  "hbm_bytes_per_launch": 1024.0 * (fetch[k] * ff + write[k] * fw)}
    if "verify" not in out and "verify_tree" in out and "verify_dense" in out:
        out["verify"] = {k: out["verify_tree"][k] + out["verify_dense"][k]
                         for k in ("fetch_kib", "write_kib", "hbm_bytes_per_launch")}
        out["verify"]["kernels"] = "tree_kernel + dense_kernel"
    out["hbm_bytes_per_launch"] = out.get("verify", {}).get("hbm_bytes_per_launch")
    with open(traffic_file(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        return "unknown"


def cpu_baseline(sets0, cfg, max_seqs, single_seqs=8):
    """The fp64 oracle as it stands (its memoised form, S_i = step(S_parent),
    bitwise equal to the per-path replay) on a bounded sample of the same
    workload: verify and commit of the first `max_seqs` sequences of input
    set 0 on the oracle's default thread count, then of the first
    `single_seqs` sequences on one thread."""
    import numpy as np
    import oracle

    nb = min(max_seqs, cfg.B)
    host = {n: sets0[n][:nb].float().cpu().numpy().astype(np.float64) for n in ("q", "k", "v", "g", "beta", "S0")}
    host["parent"] = sets0["parent"][:nb].cpu().numpy()
    acc = sets0["accepted"][:nb].cpu().numpy()
    threads = oracle.default_threads()
    # repeat the sample until about a second of wall time (about 16 s of CPU
    # work on 16 threads)
    reps, t0 = 0, time.perf_counter()
    while reps < 50 and (reps == 0 or time.perf_counter() - t0 < 1.0):
        oracle.verify_inputs(host, threads=threads)
        oracle.commit_inputs(host, accepted=acc, threads=threads)
        reps += 1
    dt = time.perf_counter() - t0
    n1 = min(single_seqs, nb)
    one = {n: a[:n1] for n, a in host.items()}
    t1 = time.perf_counter()
    oracle.verify_inputs(one, threads=1)
    oracle.commit_inputs(one, accepted=acc[:n1], threads=1)
    dt1 = time.perf_counter() - t1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": reps * nb * cfg.N * cfg.H_v / dt, "unit": "nodes·heads/s", "cores": threads,
            "host_logical_cpus": os.cpu_count(), "affinity_cpus": affinity, "cpu": host_cpu_model(),
            "kind": "oracle",
            "sample": f"fp64 oracle, memoised form (bitwise equal to its per-path replay), verify + commit "
                      f"of sequences 0..{nb - 1} of input set 0 ({nb}x{cfg.N} nodes x {cfg.H_v} heads), "
                      f"{reps} repetitions on {threads} threads (OMP_NUM_THREADS or the process's CPUs, "
                      f"at most {oracle.MAX_THREADS}), {dt:.2f} s wall",
            "single_thread": {"value": n1 * cfg.N * cfg.H_v / dt1, "unit": "nodes·heads/s", "cores": 1,
                              "sample": f"verify + commit of sequences 0..{n1 - 1}, one repetition, "
                                        f"{dt1:.2f} s wall"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="rotating input sets")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seqs", type=int, default=32, help="sequences in the CPU-oracle sample (0: skip)")
    ap.add_argument("--no-stress", action="store_true",
                    help="skip the context figure for one layer of the 48-layer N=256 stress workload")
    ap.add_argument("--kernel-only", action="store_true",
                    help="profiler runs: verify + commit back to back, then the calibration copies; "
                         "prints progress, no JSON")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of each calibration copy (--kernel-only)")
    ap.add_argument("--kernel-workload", default=WORKLOAD, choices=[WORKLOAD, STRESS],
                    help="workload of --kernel-only and --traffic-from (default: the metric's)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs of a --kernel-only run into the "
                         "per-launch HBM traffic file read by this script")
    args = ap.parse_args()

    if args.traffic_from:
        write_traffic(*args.traffic_from, copy_mib=args.copy_mib, workload=args.kernel_workload)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the verify path runs on one GPU; --gpus must be 1 "
              "(sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_tree_gdn_amd as gdn
    import gdn_inputs as G

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stress_only = args.kernel_only and args.kernel_workload == STRESS
    cfg = G.CONFIGS[STRESS if stress_only else WORKLOAD]
    gdn.load_library()

    # rotating input sets (three layers for the stress workload, seeded as in
    # its context figure below)
    sets = []
    for r in range(3 if stress_only else args.sets):
        tseed, aseed = (3000 + r, 4000 + r) if stress_only else (1000 + r, 2000 + r)
        parent = G.make_tree(cfg, G.rng_for(args.seed, tseed))
        d = G.make_inputs_device(cfg, seed=args.seed, layer=r, parent=parent, device=dev)
        d["accepted"] = torch.from_numpy(G.rng_for(args.seed, aseed).integers(0, cfg.N, size=cfg.B)
                                         .astype(np.int32)).to(dev)
        d["o"] = torch.empty((cfg.B, cfg.N, cfg.H_v, cfg.d_v), dtype=torch.float32, device=dev)
        d["S_new"] = torch.empty_like(d["S0"])
        d["ctx"] = gdn.GdnContext.for_tensors(d["q"], d["v"], d["parent"])
        sets.append(d)
    anc_depth = [G.tree_stats(s["parent"].cpu().numpy()) for s in sets]
    # path length of each accepted node (for the commit's algorithmic bytes)
    path_lens = []
    for s in sets:
        par = s["parent"].cpu().numpy()
        acc = s["accepted"].cpu().numpy()
        lens = []
        for b in range(cfg.B):
            n, x = 0, int(acc[b])
            while x >= 0:
                n += 1
                x = int(par[b, x])
            lens.append(n)
        path_lens.append(lens)

    stream = torch.cuda.current_stream()

    def verify(s):
        gdn.gdn_tree_verify(s["ctx"], s["q"], s["k"], s["v"], s["g"], s["beta"], s["parent"], s["S0"],
                            o=s["o"], stream=stream)

    def commit(s):
        gdn.gdn_commit_path(s["ctx"], s["accepted"], S_new=s["S_new"], stream=stream)

    def verify_static(s):
        gdn.gdn_tree_verify_static(s["q"], s["k"], s["v"], s["g"], s["beta"], s["parent"], s["S0"],
                                   o=s["o"], stream=stream)

    # fused commit-then-verify as a decoding chain: the tree recorded on
    # fctx (set i) is committed at its accepted nodes inside the verify of
    # set i + 1, the state alternating between two buffers
    fctx = gdn.GdnContext.for_tensors(sets[0]["q"], sets[0]["v"], sets[0]["parent"])
    fbufs = [torch.empty_like(sets[0]["S0"]) for _ in range(2)]
    fstate = {"i": 0}

    def fused_reset():
        gdn.gdn_tree_verify(fctx, sets[0]["q"], sets[0]["k"], sets[0]["v"], sets[0]["g"], sets[0]["beta"],
                            sets[0]["parent"], sets[0]["S0"], o=sets[0]["o"], stream=stream)
        fstate["i"] = 0

    def fused(_s=None):
        i = fstate["i"]
        prev, new = sets[i % len(sets)], sets[(i + 1) % len(sets)]
        gdn.gdn_commit_verify(fctx, prev["accepted"], new["q"], new["k"], new["v"], new["g"], new["beta"],
                              new["parent"], S_next=fbufs[i % 2], o=new["o"], stream=stream)
        fstate["i"] = i + 1

    if args.kernel_only:
        # each kernel back to back, as the per-kernel event timing below runs it
        # (the fused kernel serves trees of up to 128 nodes)
        if not stress_only:
            fused_reset()
        roles = (("verify", verify), ("commit", commit)) + (
            (("verify_static", verify_static),) if stress_only else (("commit_verify", fused),))
        for name, fn in roles:
            for i in range(args.warmup + args.steps):
                fn(sets[i % len(sets)])
                if i % 50 == 0:
                    torch.cuda.synchronize()
                    print(f"kernel-only: {i} {name} calls", flush=True)
            torch.cuda.synchronize()
        # calibration: a plain streaming kernel of known size (read n, write n bytes)
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_CALLS):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        print("kernel-only: done", flush=True)
        return

    for i in range(args.warmup):
        s = sets[i % len(sets)]
        verify(s)
        commit(s)
    torch.cuda.synchronize()
    for s in sets:
        gdn.gdn_ctx_status(s["ctx"])

    # --- the timed region: K verify calls -------------------------------------
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        verify(sets[i % len(sets)])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps

    def step_vc(s):
        verify(s)
        commit(s)

    # --- per-kernel averages (HIP events on the launch stream) ---------------
    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            fn(sets[i % len(sets)])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # the timed region is verify alone: its event average is the kernel's
    verify_ms = step_ms
    commit_ms = timed(commit, args.steps)
    step_vc_ms = timed(step_vc, args.steps)

    # per-call distribution: a HIP event pair around each call
    def per_call(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            fn(sets[i % len(sets)])
            b.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        return {"median_us": float(np.median(us)), "p10_us": float(np.percentile(us, 10)),
                "p90_us": float(np.percentile(us, 90)), "calls": n}

    verify_dist = per_call(verify, args.steps)
    commit_dist = per_call(commit, args.steps)
    fused_reset()
    for _ in range(args.warmup):
        fused()
    fused_ms = timed(fused, args.steps)
    fused_dist = per_call(fused, args.steps)
    gdn.gdn_ctx_status(fctx)

    # context: a plain device copy (torch), read + write of 256 MiB each
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record(stream)
    for _ in range(20):
        dst.copy_(src)
    b_ev.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 20 * 2 * src.numel() * 4 / (a_ev.elapsed_time(b_ev) * 1e-3) / 1e9
    del src, dst
    for s in sets:
        gdn.gdn_ctx_status(s["ctx"])

    nh = cfg.B * cfg.N * cfg.H_v
    vbytes = verify_bytes(cfg)
    cbytes = float(np.mean([commit_bytes(cfg, pl) for pl in path_lens]))
    fbytes = float(np.mean([commit_verify_bytes(cfg, pl) for pl in path_lens]))
    achieved = vbytes / (verify_ms * 1e-3) / 1e9
    vflops = verify_flops(cfg, float(np.mean([a["mean_strict_ancestors"] for a in anc_depth])))
    traffic = read_traffic("verify")

    # the steps around verification, and the per-branch baseline, at the
    # same workload (context, not the metric)
    def per_branch(s):
        gdn.gdn_tree_verify_branches(s["ctx"], s["q"], s["k"], s["v"], s["g"], s["beta"], s["parent"], s["S0"],
                                     o=s["o"], stream=stream)

    branch_ms = timed(per_branch, 8)
    for s in sets:
        gdn.gdn_ctx_status(s["ctx"])
    rng_t = G.rng_for(args.seed, 5000)
    root_np, node_np = G.make_candidate_logp(rng_t, cfg.B, cfg.N, 8)
    root_lp, node_lp = torch.from_numpy(root_np).to(dev), torch.from_numpy(node_np).to(dev)
    draft_np, target_np = G.make_draft_tokens(sets[0]["parent"].cpu().numpy(), rng_t)
    draft_t, target_t = torch.from_numpy(draft_np).to(dev), torch.from_numpy(target_np).to(dev)
    build_w = 8
    build_out = gdn.gdn_tree_build(root_lp, node_lp, build_w, cfg.max_depth, stream=stream)
    build_ms = timed(lambda s: gdn.gdn_tree_build(root_lp, node_lp, build_w, cfg.max_depth, stream=stream), 20)
    acc_out = gdn.gdn_accept_path(sets[0]["parent"], draft_t, target_t, stream=stream)
    accept_ms = timed(lambda s: gdn.gdn_accept_path(s["parent"], draft_t, target_t, stream=stream), 20)
    torch.cuda.synchronize()
    around = {
        "per_branch_baseline": {
            "ms": branch_ms, "nodes_heads_per_s": nh / (branch_ms * 1e-3),
            "fused_speedup": branch_ms / verify_ms, "pages_speedup_at_tree_size_128": 7.1,
            "note": "gdn_tree_verify_branches: every root-to-leaf branch stepped token by token from a fresh "
                    "copy of S0 (fp32 VALU); the pages' figure is on other hardware with their own baseline"},
        "tree_build": {"ms": build_ms, "w": build_w, "candidates": 8, "max_depth": cfg.max_depth,
                       "steps_max": int(build_out[3].max().item()),
                       "note": "gdn_tree_build, top-w best-first construction of B=32 trees of N=128 nodes"},
        "accept_path": {"ms": accept_ms,
                        "mean_accept_len": float(acc_out[1].float().mean().item()),
                        "note": "gdn_accept_path, greedy accepted-node selection over B=32 trees of N=128"},
    }
    # context (not the metric): one layer of the 48-layer stress workload,
    # trees of 256 nodes, timed the same way on three rotating layers
    stress = None
    first = sets[0]  # the CPU baseline samples it below
    n_sets = len(sets)
    if not args.no_stress:
        del sets
        torch.cuda.empty_cache()
        scfg = G.CONFIGS["stress48"]
        ssets = []
        for r in range(3):
            parent = G.make_tree(scfg, G.rng_for(args.seed, 3000 + r))
            d = G.make_inputs_device(scfg, seed=args.seed, layer=r, parent=parent, device=dev)
            d["accepted"] = torch.from_numpy(G.rng_for(args.seed, 4000 + r).integers(0, scfg.N, size=scfg.B)
                                             .astype(np.int32)).to(dev)
            d["o"] = torch.empty((scfg.B, scfg.N, scfg.H_v, scfg.d_v), dtype=torch.float32, device=dev)
            d["S_new"] = torch.empty_like(d["S0"])
            d["ctx"] = gdn.GdnContext.for_tensors(d["q"], d["v"], d["parent"])
            ssets.append(d)
        sets = ssets
        for i in range(6):
            verify(sets[i % 3])
            commit(sets[i % 3])
        torch.cuda.synchronize()
        sv_ms, sc_ms = timed(verify, 30), timed(commit, 30)
        for i in range(3):
            verify_static(sets[i % 3])
        torch.cuda.synchronize()
        ss_ms = timed(verify_static, 30)
        for s in sets:
            gdn.gdn_ctx_status(s["ctx"])
        sb = verify_bytes(scfg)
        stress = {"workload": "stress48 layer (B=64, N=256, H_v=32, H_k=16, d=128, depth<=24)",
                  "verify_us": sv_ms * 1e3, "commit_us": sc_ms * 1e3, "verify_algorithmic_bytes": sb,
                  "verify_GBps": sb / (sv_ms * 1e-3) / 1e9, "verify_frac_of_peak": sb / (sv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "verify_traffic": read_traffic("verify", STRESS),
                  "verify_kernels": "tree_kernel, then dense_kernel (two launches over the context's workspace)",
                  "static_verify_us": ss_ms * 1e3,
                  "static_verify_frac_of_peak": sb / (ss_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "static_verify_traffic": read_traffic("verify_static", STRESS),
                  "static_verify_kernel": "verify_fast_kernel (gdn_tree_verify_static: no context, no workspace)",
                  "verify_nodes_heads_per_s": scfg.B * scfg.N * scfg.H_v / (sv_ms * 1e-3)}
        del ssets, sets
        torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": nh / (step_ms * 1e-3),
        "unit": "nodes·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded best-first trees and N(0,1)-derived tensors; no model weights)",
        "config": {"workload": WORKLOAD, "B": cfg.B, "N": cfg.N, "H_k": cfg.H_k, "H_v": cfg.H_v,
                   "d_k": cfg.d_k, "d_v": cfg.d_v, "qkv": cfg.dtype, "state": "f32", "output": "f32",
                   "tree": f"best_first depth<={cfg.max_depth}",
                   "mean_strict_ancestors": float(np.mean([a["mean_strict_ancestors"] for a in anc_depth])),
                   "max_depth": int(max(a["max_depth"] for a in anc_depth)),
                   "rotating_sets": n_sets, "timed_call": "gdn_tree_verify",
                   "arithmetic": "bf16 MFMA with fp32 accumulation; fp32 operands as bf16 hi+lo pairs; "
                                 "fp32 VALU for gates and the triangular solves"},
        "verify": {"ms": verify_ms, "nodes_heads_per_s": nh / (verify_ms * 1e-3),
                   "algorithmic_bytes": vbytes, "GBps": achieved, "per_call": verify_dist},
        "step_verify_commit": {"ms": step_vc_ms, "nodes_heads_per_s": nh / (step_vc_ms * 1e-3),
                               "note": "gdn_tree_verify then gdn_commit_path, back to back"},
        "step_commit_verify_fused": {
            "ms": fused_ms, "per_call": fused_dist, "algorithmic_bytes": fbytes,
            "GBps": fbytes / (fused_ms * 1e-3) / 1e9, "frac": fbytes / (fused_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "speedup_vs_separate": step_vc_ms / fused_ms, "traffic": read_traffic("commit_verify"),
            "note": "gdn_commit_verify: the previous tree's commit at its accepted nodes formed on chip inside "
                    "the next tree's verify, the committed state written once and not read back"},
        "commit": {"ms": commit_ms, "per_call": commit_dist, "algorithmic_bytes": cbytes,
                   "GBps": cbytes / (commit_ms * 1e-3) / 1e9,
                   "frac": cbytes / (commit_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": read_traffic("commit")},
        "roofline": {"bound": "hbm", "kernel": "gdn_tree_verify", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic},
        "mfma_secondary": {"kernel": "gdn_tree_verify", "algorithmic_flop": vflops,
                           "achieved": vflops / (verify_ms * 1e-3) / 1e12, "peak": BF16_MFMA_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": vflops / (verify_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS},
        "device_copy": {"GBps": copy_gbps, "bytes_per_copy": 2 * (64 << 20) * 4,
                        "note": "torch copy_ of 256 MiB, read + write; context for the 8 TB/s peak"},
        "context_stress_layer": stress,
        "around_verify": around,
        "wall_s_timed_region": wall,
    }
    if args.cpu_seqs > 0:
        out["cpu_baseline"] = cpu_baseline(first, cfg, args.cpu_seqs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
