"""Benchmark of the draft-tree construction hot path on one MI355X.

One step = one pass of the whole hot path over a batch of R = 64 rounds
(L = 16 draft positions, V = 151,936, bf16 logits, synthetic seeded inputs):
  1. build_tree_marginal   DDTree-shape logits, K = B = 64, beta = 0
  2. build_tree_depthwise  same logits as base, Markov head E 151936x1024, U 16x1024x64,
                           P 64x151936, K = 8, W = 32, B = 128, beta = -0.5
  3. build_tree_gated      TALON-shape logits, K_root = 10, mu = 0.03, N = 60
  4. accept_tree T = 0     the step's marginal trees against draft-correlated target logits
  5. accept_tree T = 1     same, one Philox-seeded trial per round (trial index = step)
Timed outside the step and reported under extra_ms: the matching walk, DARTree's exact
(W = B) and fixed (W = B / L) widths, the static D x K grid (K = 10, D = 6) and GRAFT's
edge-scored best-first tree (K = 32, B = 128).
value = rounds per second of that whole step (R / step time). Inputs are resident in
HBM before timing. Prints one JSON line.

The roofline object is for the logits row sweep (fused log-softmax + top-K), the
kernel every builder runs over its [R, L, V] logits, timed live with HIP events over
K launches of dtree_topk_logsoftmax on the same stream; algorithmic bytes per launch
= R*L*V*2 (each bf16 logit read once) + the K-list outputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

R, L, V = 64, 16, 151936
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "rowsweep_traffic.json"))
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run 5 row sweeps and 5 plain copies of the same bytes (for rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE runs: the copy calibrates the counters)")
    return ap.parse_args()


def sweep_source_digest():
    """Digest of the row sweep's sources (the kernel and the helpers it includes): the stored
    counter readings are used only while it matches."""
    import hashlib
    h = hashlib.sha256()
    for f in ("k_rowsweep.hip", "common.hpp"):
        h.update(open(os.path.join(ROOT, "draft_tree_construction_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(rounds shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import draft_tree_construction_amd as dt
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.traffic_probe:
        traffic_probe(dt, synth, torch, np, dev)
        return

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs (seeded, resident in HBM)
    draft_h = synth.ddtree_logits(seed=2)
    draft = bf(draft_h)
    talon_h = synth.talon_logits(seed=4)
    talon = bf(talon_h)
    head = synth.correction_head(seed=3)
    E_h, U_h, P_h, root_h = head
    E, U, P = bf(E_h), bf(U_h), bf(P_h)
    root = torch.from_numpy(root_h).to(dev)

    ws_m = torch.empty(dt.workspace_size(dt.OP_MARGINAL, R, L, V, 64, 64), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(dt.workspace_size(dt.OP_DEPTHWISE, R, L, V, 8, 128, 32, 64, 1024), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(dt.workspace_size(dt.OP_GATED, R, L, V, 0, 60), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(dt.workspace_size(dt.OP_ACCEPT, R, L, V, 0, 64), dtype=torch.uint8, device=dev)
    t_m, t_d, t_g = dt.Tree.empty(R, 64, dev), dt.Tree.empty(R, 128, dev), dt.Tree.empty(R, 60, dev)
    o0 = tuple(torch.empty(1, R, dtype=torch.int32, device=dev) for _ in range(3))
    o1 = tuple(torch.empty(1, R, dtype=torch.int32, device=dev) for _ in range(3))

    # target logits follow the marginal trees' depths (deterministic, so built once)
    dt.build_tree_marginal(draft, 64, 64, 0.0, ws=ws_m, out=t_m)
    torch.cuda.synchronize()
    target = bf(synth.verification_target(draft_h, t_m.depth.cpu().numpy(), seed=5))

    stream = torch.cuda.current_stream(dev)
    names = ["marginal", "depthwise", "gated", "accept_t0", "accept_t1"]

    def step(i, ev=None):
        def mark(k):
            if ev is not None:
                ev[k].record(stream)
        mark(0)
        dt.build_tree_marginal(draft, 64, 64, 0.0, ws=ws_m, out=t_m)
        mark(1)
        dt.build_tree_depthwise(draft, E, U, P, root, 8, 32, 128, -0.5, ws=ws_d, out=t_d)
        mark(2)
        dt.build_tree_gated(talon, 10, 0.03, 60, ws=ws_g, out=t_g)
        mark(3)
        dt.accept_tree(t_m, target, None, 0.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o0)
        mark(4)
        dt.accept_tree(t_m, target, draft, 1.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o1)
        mark(5)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, synchronised on both sides
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[evs[i][k].elapsed_time(evs[i][k + 1]) for k in range(5)] for i in range(args.steps)])
    step_ms = float(np.sum(per, axis=1).mean())
    ms_per_step = wall * 1e3 / args.steps
    value = R / (ms_per_step / 1e3)

    # ---- roofline: the row sweep kernel, timed live over its own launches on this stream
    flat = draft.view(R * L, V)
    K = 64
    lse = torch.empty(R * L, dtype=torch.float32, device=dev)
    ids = torch.empty(R * L, K, dtype=torch.int32, device=dev)
    lp = torch.empty(R * L, K, dtype=torch.float32, device=dev)
    ws_t = torch.empty(max(dt.workspace_size(dt.OP_TOPK, R * L, 1, V, K), 1), dtype=torch.uint8, device=dev)
    for _ in range(3):
        dt.topk_logsoftmax(flat, K, ws=ws_t)
    torch.cuda.synchronize()
    n_sweep = max(args.steps, 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_sweep):
        dt.lib().dtree_topk_logsoftmax(flat.data_ptr(), 0, R * L, V, K, lse.data_ptr(), ids.data_ptr(),
                                       lp.data_ptr(), ws_t.data_ptr(), ws_t.numel(), stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    sweep_us = e0.elapsed_time(e1) * 1e3 / n_sweep
    alg_bytes = R * L * V * 2 + R * L * (4 + K * 8)
    achieved = alg_bytes / (sweep_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            rec = json.load(open(args.traffic_json))
            if rec.get("source_digest") == sweep_source_digest():
                traffic = rec.get("bytes_per_launch")
        except Exception:
            traffic = None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_rowsweep<bf16> (dtree_topk_logsoftmax, R*L=1024 rows, K=64)",
                "us_per_launch": round(sweep_us, 2), "alg_bytes_per_launch": alg_bytes}

    # ---- outside the step: exact target-sample matching (T = 1, one trial per round) on the
    # same trees and target rows, timed per call with events on this stream
    ws_x = torch.empty(dt.workspace_size(dt.OP_ACCEPT, R, 1, V, 0, 64), dtype=torch.uint8, device=dev)
    for i in range(3):
        dt.accept_tree_match(t_m, target, 1.0, synth.PHILOX_SEED, i, 1, ws=ws_x, outs=o1)
    torch.cuda.synchronize()
    n_match = max(args.steps, 10)
    ex = [torch.cuda.Event(enable_timing=True) for _ in range(n_match + 1)]
    ex[0].record(stream)
    for i in range(n_match):
        dt.accept_tree_match(t_m, target, 1.0, synth.PHILOX_SEED, i, 1, ws=ws_x, outs=o1)
        ex[i + 1].record(stream)
    torch.cuda.synchronize()
    match_ms = float(np.mean([ex[i].elapsed_time(ex[i + 1]) for i in range(n_match)]))

    # ---- outside the step: DARTree's other widths on the same inputs, W = B (the exact
    # best-first tree) and W = B / L (the fixed variant), beta = 0; and each tree's covered
    # draft mass, sum over nodes of exp(s_0(u)) (s_0 the score without the depth bonus; the
    # expected accepted length under the corrected draft, DDTree's Proposition 1)
    def covered(t, beta):
        sc, dp = t.score.cpu().numpy().astype(np.float64), t.depth.cpu().numpy()
        nn = t.n_nodes.cpu().numpy()
        return float(np.mean([np.exp(sc[r, 1:nn[r] + 1] - beta * dp[r, 1:nn[r] + 1]).sum() for r in range(R)]))

    ws_w = torch.empty(dt.workspace_size(dt.OP_DEPTHWISE, R, L, V, 8, 128, 128, 64, 1024), dtype=torch.uint8,
                       device=dev)
    t_w = dt.Tree.empty(R, 128, dev)
    extra_ms = {"accept_match_t1": round(match_ms, 4)}
    mass = {"pruned_w32_beta-0.5": round(covered(t_d, -0.5), 4)}
    for name, W in (("exact_w128", 128), ("fixed_w8", 8)):
        for _ in range(2):
            dt.build_tree_depthwise(draft, E, U, P, root, 8, W, 128, 0.0, ws=ws_w, out=t_w)
        torch.cuda.synchronize()
        ew = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ew[0].record(stream)
        for i in range(5):
            dt.build_tree_depthwise(draft, E, U, P, root, 8, W, 128, 0.0, ws=ws_w, out=t_w)
            ew[i + 1].record(stream)
        torch.cuda.synchronize()
        extra_ms["depthwise_" + name] = round(float(np.mean([ew[i].elapsed_time(ew[i + 1]) for i in range(5)])), 4)
        mass[name] = round(covered(t_w, 0.0), 4)

    # ---- outside the step: the static D x K grid, K = 10, D = 6 (60 nodes, TALON's budget N),
    # on the TALON-shape logits: the fixed-shape builder of TALON's tree-build comparison,
    # next to the step's gated tree (its time is breakdown_ms["gated"])
    t_s = dt.Tree.empty(R, 60, dev)
    ws_s = torch.empty(dt.workspace_size(dt.OP_STATIC, R, L, V, 10), dtype=torch.uint8, device=dev)
    for _ in range(2):
        dt.build_tree_static(talon, 10, 6, ws=ws_s, out=t_s)
    torch.cuda.synchronize()
    es = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    es[0].record(stream)
    for i in range(5):
        dt.build_tree_static(talon, 10, 6, ws=ws_s, out=t_s)
        es[i + 1].record(stream)
    torch.cuda.synchronize()
    extra_ms["static_k10_d6"] = round(float(np.mean([es[i].elapsed_time(es[i + 1]) for i in range(5)])), 4)
    mass["talon_gated_n60"] = round(covered(t_g, 0.0), 4)
    mass["static_k10_d6"] = round(covered(t_s, 0.0), 4)

    # ---- outside the step: GRAFT's edge-scored best-first tree on the DDTree-shape logits,
    # K = 32 candidates per position, B = 128, random-init edge MLP (hp = hc = 64, hd = 16,
    # H = 128)
    prm, root_g = synth.edge_mlp(seed=6)
    mlp = {k: torch.from_numpy(prm[k]).to(dev) for k in ("Gp", "Gc", "Ed", "W", "b", "w")}
    mlp["b0"], mlp["s"] = prm["b0"], prm["s"]
    root_g = torch.from_numpy(root_g).to(dev)
    t_t = dt.Tree.empty(R, 128, dev)
    ws_e = torch.empty(dt.workspace_size(dt.OP_TDES, R, L, V, 32), dtype=torch.uint8, device=dev)
    for _ in range(2):
        dt.build_tree_tdes(draft, root_g, mlp, 32, 128, ws=ws_e, out=t_t)
    torch.cuda.synchronize()
    es = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    es[0].record(stream)
    for i in range(5):
        dt.build_tree_tdes(draft, root_g, mlp, 32, 128, ws=ws_e, out=t_t)
        es[i + 1].record(stream)
    torch.cuda.synchronize()
    extra_ms["tdes_k32_b128"] = round(float(np.mean([es[i].elapsed_time(es[i + 1]) for i in range(5)])), 4)

    out = {
        "metric": "tree-build rounds/sec + us/round at V=151936,L=16,B=128; HBM GB/s vs peak",
        "value": round(value, 1), "unit": "rounds/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "us_per_round": round(ms_per_step * 1e3 / R, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "R=64 rounds, L=16, V=151936 bf16: marginal K=B=64 + depthwise K=8,W=32,B=128,"
                               "beta=-0.5,E 151936x1024,rank 64 + gated K_root=10,mu=0.03,N=60 + "
                               "accept T=0 and T=1 (1 trial/round) on the marginal trees",
                   "rounds": R, "L": L, "V": V},
        "breakdown_us_per_round": {n: round(float(per[:, k].mean()) * 1e3 / R, 3) for k, n in enumerate(names)},
        "breakdown_ms": {n: round(float(per[:, k].mean()), 4) for k, n in enumerate(names)},
        "event_ms_per_step": round(step_ms, 4),
        "roofline": roofline,
        "extra_ms": extra_ms,
        "covered_draft_mass": mass,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(draft_h, talon_h, head)
    print(json.dumps(out), flush=True)


def traffic_probe(dt, synth, torch, np, dev):
    """5 row sweeps over the [R*L, V] bf16 logits (K = 64), then 5 device-to-device copies of
    a buffer of the same size: the copy reads and writes exactly R*L*V*2 bytes, which scales
    the counters' readings to bytes."""
    bits = synth.ddtree_logits(seed=2)
    flat = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev).view(R * L, V)
    K = 64
    ws_t = torch.empty(max(dt.workspace_size(dt.OP_TOPK, R * L, 1, V, K), 1), dtype=torch.uint8, device=dev)
    for _ in range(5):
        dt.topk_logsoftmax(flat, K, ws=ws_t)
    dst = torch.empty_like(flat)
    for _ in range(5):
        dst.copy_(flat)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "rowsweep+copy", "copy_bytes_each_way": R * L * V * 2,
                      "source_digest": sweep_source_digest()}), flush=True)


def cpu_baseline(draft_h, talon_h, head, n_rounds=16):
    """The oracle, as it stands, on a bounded sample: the first `n_rounds` rounds of the same
    step (all five operations, each round's own inputs), float64 numpy on one thread."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import synth
    from oracle import accept, depthwise, gated, marginal, rowsweep

    ctx = threadpool_limits(1) if threadpool_limits else None
    try:
        E_h, U_h, P_h, root_h = head
        U64 = synth.f32_from_bf16(U_h).astype(np.float64)
        P64 = synth.f32_from_bf16(P_h).astype(np.float64)

        class Rows:  # rows of E gathered on demand
            def __getitem__(self, idx):
                return synth.f32_from_bf16(E_h[idx]).astype(np.float64)

        elapsed = 0.0
        for r in range(n_rounds):
            z = rowsweep.as_f64(draft_h[r], "bf16")
            tal = rowsweep.as_f64(talon_h[r], "bf16")
            t0 = time.perf_counter()
            tm = marginal.build_marginal(z, 64, 64, 0.0)
            depthwise.build_depthwise(z, Rows(), U64, P64, int(root_h[r]), 8, 32, 128, -0.5)
            gated.build_gated(tal, 10, float(np.float32(0.03)), 60, full_pool=False)
            elapsed += time.perf_counter() - t0
            # the target rows follow this round's marginal tree (input preparation, untimed)
            depth = np.array(tm.arrays(64)[2])[None, :]
            tgt = rowsweep.as_f64(synth.verification_target(draft_h[r:r + 1], depth, seed=5)[0], "bf16")
            t0 = time.perf_counter()
            accept.walk_greedy(tm.parent, tm.token, tm.depth, tgt[:tm.n + 1])
            tab = accept.ResidualTables(tm.parent, tm.token, tm.depth, tgt[:tm.n + 1], z, 1.0)
            accept.walk_sampled(tab, tm.depth, synth.PHILOX_SEED, 0, r)
            elapsed += time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": round(n_rounds / elapsed, 4), "unit": "rounds/s", "cores": 1, "kind": "oracle",
            "sample": f"rounds 0..{n_rounds - 1} of the full step (marginal + depthwise + gated + accept T=0 "
                      f"+ T=1 per round), float64 numpy, 1 thread; {elapsed:.2f} s"}


if __name__ == "__main__":
    main()
