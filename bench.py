"""Benchmark of the draft-tree construction hot path on one MI355X.

One step = one pass of the whole hot path over a batch of R = 64 rounds
(L = 16 draft positions, V = 151,936, bf16 logits, synthetic seeded inputs):
  0. dtree_topk_lists      the row sweep of the DDTree-shape logits, K = 64, once: both
                           builders of those logits take their candidates from it
  1. build_tree_marginal_lists   K = B = 64, beta = 0
  2. build_tree_depthwise_lists  the same logits as base (C_d = the first 8 of each list),
                           Markov head E 151936x1024, U 16x1024x64, P 64x151936 (its
                           transposes prepared once before timing, as constant weights are),
                           K = 8, W = 32, B = 128, beta = -0.5
  3. build_tree_gated      TALON-shape logits (its own sweep), K_root = 10, mu = 0.03, N = 60
  4. accept_tree_narrow T = 0   the step's marginal trees against draft-correlated target
                           logits (one workgroup per round: the walks run beside the
                           depth-wise builder, so they take a CU per round, not four)
  5. accept_tree_narrow T = 1   same, one Philox-seeded trial per round (trial index = step)
  (in the overlapped step the T = 1 walk runs before the T = 0 walk on the main stream)
Each configuration's builder as a user calls it alone (its own sweep included) is timed too:
per_config_ms, the median of as many calls as timed steps; the walks there are accept_tree
(four workgroups per round, the lower latency for a call that has the device to itself).
Timed outside the step and reported under extra_ms: the matching walk, DARTree's exact
(W = B) and fixed (W = B / L) widths, the static D x K grid (K = 10, D = 6) and GRAFT's
edge-scored best-first tree (K = 32, B = 128).
value = rounds per second of that whole step (R / step time). The step's independent parts
run concurrently on three streams of default priority: 0 -> 1 -> 4 -> 5 on the main one
(the walks need the marginal trees), 2 on a second once the lists are written, 3 on a third
from the start, all joined at the end of every step; the per-operation breakdown comes from
the same work serialised on one stream after the timed region (breakdown_ms: the median per
operation over as many serialised steps as timed steps; breakdown_ms_mean the mean). Inputs are resident in HBM before timing. Prints one
JSON line.

The roofline object is for the logits row sweep (fused log-softmax + top-K), the
kernel every builder runs over its [R, L, V] logits, timed live with HIP events over
K launches of dtree_topk_logsoftmax on the same stream; algorithmic bytes per launch
= R*L*V*2 (each bf16 logit read once) + the K-list outputs; traffic_gbps is the counter
bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled) over the same launch time.
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "rowsweep_traffic.json"))
    ap.add_argument("--step-only", action="store_true",
                    help="run only the warm-up and timed steps, serialised on one stream, and print their line "
                         "(for profiler passes: no roofline sweeps, extra builders, single-round latencies or cpu leg)")
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


def depthwise_source_digest():
    """Digest of the depth-wise kernels' sources: the stored counter readings of the correction
    sweep are used only while it matches."""
    import hashlib
    h = hashlib.sha256()
    for f in ("k_depthwise.hip", "common.hpp"):
        h.update(open(os.path.join(ROOT, "draft_tree_construction_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


# Issue cost of one wave64 vector instruction on a gfx950 SIMD, measured with a throughput
# probe (eight independent chains per lane, eight waves per SIMD, every CU busy; cycles at
# the 2.4 GHz clock the device reports): v_add_f32 / v_fma_f32 2.9-3.1 cycles, v_exp_f32 9.6.
VALU_CYC, TRANS_CYC = 3.0, 9.6


def correction_gemm(path, K=8):
    """The depth-wise correction sweep (k_dw_corr) against its ceilings, from the rocprofv3
    readings stored with the source digest: MFMA utilisation of the algorithmic h . P product
    (live states x 2 x rank x V flop) at the traced kernel time, the matrix cores' busy
    fraction, and the vector-issue floor from the instruction counts at the measured issue
    costs (VALU_CYC, TRANS_CYC; 1024 SIMDs at 2.4 GHz). None when the readings are missing
    or stale."""
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_digest") != depthwise_source_digest():
        return None
    c = rec["per_dispatch"]
    t = rec["trace_us_mean"] * 1e-6
    simd_cycles = 1024 * 2.4e9
    live = R * (1 + (L - 1) * K)
    alg_flops = live * 2 * 64 * V
    trans = c["SQ_INSTS_VALU_TRANS_F32"]
    exp_floor = trans * TRANS_CYC / simd_cycles
    valu_floor = ((c["SQ_INSTS_VALU"] - trans) * VALU_CYC + trans * TRANS_CYC) / simd_cycles
    return {"kernel": "k_dw_corr<bf16>", "us_per_launch": rec["trace_us_mean"], "source": os.path.relpath(path, ROOT),
            "alg_flops": alg_flops, "mfma_util": round(alg_flops / t / 2.5e15, 4),
            "mfma_busy": round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (simd_cycles * t), 4),
            "exps": trans * 64, "exp_floor_us": round(exp_floor * 1e6, 1),
            "valu_issue_floor_us": round(valu_floor * 1e6, 1), "frac_of_valu_floor": round(valu_floor / t, 4),
            "valu_cycles_per_wave_instr": VALU_CYC, "trans_cycles_per_wave_instr": TRANS_CYC,
            "bound": "neither issue floor: VALU and MFMA pipes both part-idle (per-block barrier, LDS and MFMA latencies)"}


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
    ws_d = torch.empty(dt.workspace_size(dt.OP_DEPTHWISE_PREPARED, R, L, V, 8, 128, 32, 64, 1024), dtype=torch.uint8,
                       device=dev)
    ws_dl = torch.empty(dt.workspace_size(dt.OP_DEPTHWISE_LISTS, R, L, V, 8, 128, 32, 64, 1024), dtype=torch.uint8,
                        device=dev)
    lists = dt.Lists.empty(R * L, 64, dev)  # the draft logits' candidate lists, shared by two builders
    ws_l = torch.empty(max(dt.workspace_size(dt.OP_TOPK, R * L, 1, V, 64), 1), dtype=torch.uint8, device=dev)
    head_d = dt.prepare_depthwise_head(U, P)  # constant weights: transposed once
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
    names = ["row_sweep_draft", "marginal", "depthwise", "gated", "accept_t0", "accept_t1"]
    # the step's schedule: the draft logits' row sweep, the marginal tree from its lists and
    # the two walks on that tree (T = 1, then T = 0; a chain) on the main stream; the depth-wise tree from the
    # same lists on a second stream once they are written; the gated tree (other logits, its
    # own sweep) on a third from the start; joined at the end. Of the orders tried this one
    # finished soonest.
    s_dw, s_g = torch.cuda.Stream(dev), torch.cuda.Stream(dev)

    def step_overlap(i):
        fork = torch.cuda.Event()
        fork.record(stream)
        s_g.wait_event(fork)
        with torch.cuda.stream(s_g):
            dt.build_tree_gated(talon, 10, 0.03, 60, ws=ws_g, out=t_g)
        dt.topk_lists(draft, 64, ws=ws_l, out=lists)
        have_lists = torch.cuda.Event()
        have_lists.record(stream)
        s_dw.wait_event(have_lists)
        with torch.cuda.stream(s_dw):
            dt.build_tree_depthwise_lists(draft, lists, E, head_d, 1024, 64, root, 8, 32, 128, -0.5, ws=ws_dl,
                                          out=t_d)
        dt.build_tree_marginal_lists(lists, R, L, 64, 0.0, out=t_m)
        # the longer walk first: it then overlaps more of the side streams' work
        dt.accept_tree_narrow(t_m, target, draft, 1.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o1)
        dt.accept_tree_narrow(t_m, target, None, 0.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o0)
        for s2 in (s_dw, s_g):
            join = torch.cuda.Event()
            join.record(s2)
            stream.wait_event(join)

    def step(i, ev=None):
        def mark(k):
            if ev is not None:
                ev[k].record(stream)
        mark(0)
        dt.topk_lists(draft, 64, ws=ws_l, out=lists)
        mark(1)
        dt.build_tree_marginal_lists(lists, R, L, 64, 0.0, out=t_m)
        mark(2)
        dt.build_tree_depthwise_lists(draft, lists, E, head_d, 1024, 64, root, 8, 32, 128, -0.5, ws=ws_dl, out=t_d)
        mark(3)
        dt.build_tree_gated(talon, 10, 0.03, 60, ws=ws_g, out=t_g)
        mark(4)
        dt.accept_tree_narrow(t_m, target, None, 0.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o0)
        mark(5)
        dt.accept_tree_narrow(t_m, target, draft, 1.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o1)
        mark(6)

    # (profiler passes run the serialised step only: device-wide counters of one dispatch
    # must not include kernels of the other streams)
    run = step if args.step_only else step_overlap
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, synchronised on both sides
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = R / (ms_per_step / 1e3)
    # every walk of the last timed step finished (a failed walk reports -1)
    walk_failures = int((o0[0] < 0).sum().item() + (o1[0] < 0).sum().item())
    # the same work serialised on one stream, timed per operation with HIP events (outside
    # the timed region): the per-operation breakdown
    n_ser = 2 if args.step_only else max(5, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(n_ser)]
    for i in range(n_ser):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    per = np.array([[evs[i][k].elapsed_time(evs[i][k + 1]) for k in range(len(names))] for i in range(n_ser)])
    step_ms = float(np.sum(per, axis=1).mean())
    if args.step_only:
        print(json.dumps({"metric": "tree-build rounds/sec (step serialised, profiler pass)", "value": round(value, 1),
                          "unit": "rounds/s", "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": round(ms_per_step, 4),
                          "breakdown_ms": {n: round(float(np.median(per[:, k])), 4) for k, n in enumerate(names)}}),
              flush=True)
        return

    # ---- each configuration's builder (and the two walks) as a user calls it on its own,
    # row sweep included: events around every call, the median of n_ser calls
    def cfg_marginal(i):
        dt.build_tree_marginal(draft, 64, 64, 0.0, ws=ws_m, out=t_m)

    def cfg_depthwise(i):
        dt.build_tree_depthwise_prepared(draft, E, head_d, 1024, 64, root, 8, 32, 128, -0.5, ws=ws_d, out=t_d)

    def cfg_gated(i):
        dt.build_tree_gated(talon, 10, 0.03, 60, ws=ws_g, out=t_g)

    def cfg_t0(i):
        dt.accept_tree(t_m, target, None, 0.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o0)

    def cfg_t1(i):
        dt.accept_tree(t_m, target, draft, 1.0, synth.PHILOX_SEED, i, 1, ws=ws_a, outs=o1)

    per_config = {}
    for name, f in (("cfg2_marginal", cfg_marginal), ("cfg3_depthwise", cfg_depthwise), ("cfg4_gated", cfg_gated),
                    ("cfg5_accept_t0", cfg_t0), ("cfg5_accept_t1", cfg_t1)):
        for i in range(3):
            f(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ser + 1)]
        ev[0].record(stream)
        for i in range(n_ser):
            f(args.warmup + i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per_config[name] = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(n_ser)]))

    # ---- roofline: the row sweep kernel, timed live over its own launches on this stream,
    # alternating between two distinct 311 MB logits tensors (the DDTree-shape and TALON-shape
    # inputs) so no launch re-reads what the previous one left in the 256 MB last-level cache
    flats = (draft.view(R * L, V), talon.view(R * L, V))
    K = 64
    lse = torch.empty(R * L, dtype=torch.float32, device=dev)
    ids = torch.empty(R * L, K, dtype=torch.int32, device=dev)
    lp = torch.empty(R * L, K, dtype=torch.float32, device=dev)
    ws_t = torch.empty(max(dt.workspace_size(dt.OP_TOPK, R * L, 1, V, K), 1), dtype=torch.uint8, device=dev)
    for i in range(4):
        dt.topk_logsoftmax(flats[i % 2], K, ws=ws_t)
    torch.cuda.synchronize()

    def sweep_us(n, alternate):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            x = flats[i % 2 if alternate else 0]
            dt.lib().dtree_topk_logsoftmax(x.data_ptr(), 0, R * L, V, K, lse.data_ptr(), ids.data_ptr(),
                                           lp.data_ptr(), ws_t.data_ptr(), ws_t.numel(), stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    n_sweep = max(2 * args.steps, 20)
    sweep_alt = sweep_us(n_sweep, True)
    sweep_same = sweep_us(n_sweep, False)
    alg_bytes = R * L * V * 2 + R * L * (4 + K * 8)
    achieved = alg_bytes / (sweep_alt * 1e-6) / 1e9
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
                "traffic_gbps": round(traffic / (sweep_alt * 1e-6) / 1e9, 1) if traffic else None,
                "kernel": "k_rowsweep<bf16> (dtree_topk_logsoftmax, R*L=1024 rows, K=64)",
                "us_per_launch": round(sweep_alt, 2), "alg_bytes_per_launch": alg_bytes,
                "launches": "alternating two distinct 311 MB tensors",
                "us_per_launch_same_tensor": round(sweep_same, 2)}

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

    def timed(fn, n=5):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ew = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ew[0].record(stream)
        for i in range(n):
            fn()
            ew[i + 1].record(stream)
        torch.cuda.synchronize()
        return round(float(np.mean([ew[i].elapsed_time(ew[i + 1]) for i in range(n)])), 4)

    for name, W in (("exact_w128", 128), ("fixed_w8", 8)):
        extra_ms["depthwise_" + name] = timed(lambda: dt.build_tree_depthwise_prepared(
            draft, E, head_d, 1024, 64, root, 8, W, 128, 0.0, ws=ws_w, out=t_w))
        mass[name] = round(covered(t_w, 0.0), 4)
    # the same exact tree built one node at a time: DARTree's sequential correction with a heap
    # (one correction sweep per popped node, B = 128 dependent steps, the rounds batched per step)
    ws_q = torch.empty(dt.workspace_size(dt.OP_SEQUENTIAL, R, L, V, 8, 128, 0, 64, 1024), dtype=torch.uint8,
                       device=dev)
    t_q = dt.Tree.empty(R, 128, dev)
    extra_ms["sequential_exact_b128"] = timed(lambda: dt.build_tree_sequential(
        draft, E, head_d, 1024, 64, root, 8, 128, 0.0, ws=ws_q, out=t_q), n=3)
    mass["sequential_exact_b128"] = round(covered(t_q, 0.0), 4)
    # the builder that also transposes the head on every call (build_tree_depthwise), W = 32
    extra_ms["depthwise_w32_unprepared_head"] = timed(lambda: dt.build_tree_depthwise(
        draft, E, U, P, root, 8, 32, 128, -0.5, ws=ws_w, out=t_w))
    extra_ms["prepare_depthwise_head"] = timed(lambda: dt.prepare_depthwise_head(U, P, head=head_d))
    # the step's walks (one workgroup per round) each called alone
    extra_ms["accept_t0_narrow"] = timed(lambda: dt.accept_tree_narrow(t_m, target, None, 0.0, synth.PHILOX_SEED, 7,
                                                                       1, ws=ws_a, outs=o0))
    extra_ms["accept_t1_narrow"] = timed(lambda: dt.accept_tree_narrow(t_m, target, draft, 1.0, synth.PHILOX_SEED, 7,
                                                                       1, ws=ws_a, outs=o1))

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

    # ---- single-round latency (R = 1): each builder and walk on the first round's inputs, the
    # median over 50 calls of HIP events around the call (the GRAFT figure it compares with is
    # a per-round overhead below 0.5 ms)
    def one(t, cap):
        return dt.Tree(*(x[0:1] for x in (t.parent, t.token, t.depth, t.score, t.mask, t.n_nodes)), cap)

    r1 = dict(draft=draft[0:1], talon=talon[0:1], target=target[0:1], root=root[0:1], root_g=root_g[0:1])
    tm1, td1, tg1, ts1, tt1 = (dt.Tree.empty(1, c, dev) for c in (64, 128, 60, 60, 128))
    o1r = tuple(torch.empty(1, 1, dtype=torch.int32, device=dev) for _ in range(3))
    w1 = {k: torch.empty(max(dt.workspace_size(*a), 1), dtype=torch.uint8, device=dev) for k, a in dict(
        m=(dt.OP_MARGINAL, 1, L, V, 64, 64), d=(dt.OP_DEPTHWISE_PREPARED, 1, L, V, 8, 128, 32, 64, 1024),
        g=(dt.OP_GATED, 1, L, V, 0, 60), s=(dt.OP_STATIC, 1, L, V, 10), e=(dt.OP_TDES, 1, L, V, 32),
        a=(dt.OP_ACCEPT, 1, L, V, 0, 64), q=(dt.OP_SEQUENTIAL, 1, L, V, 8, 128, 0, 64, 1024),
        x=(dt.OP_DEPTHWISE_PREPARED, 1, L, V, 8, 128, 128, 64, 1024)).items()}
    tq1, tx1 = dt.Tree.empty(1, 128, dev), dt.Tree.empty(1, 128, dev)
    tm_1 = one(t_m, 64)
    ops1 = {
        "marginal": lambda i: dt.build_tree_marginal(r1["draft"], 64, 64, 0.0, ws=w1["m"], out=tm1),
        "depthwise": lambda i: dt.build_tree_depthwise_prepared(r1["draft"], E, head_d, 1024, 64, r1["root"], 8, 32,
                                                                128, -0.5, ws=w1["d"], out=td1),
        "depthwise_exact_w128": lambda i: dt.build_tree_depthwise_prepared(
            r1["draft"], E, head_d, 1024, 64, r1["root"], 8, 128, 128, 0.0, ws=w1["x"], out=tx1),
        "sequential_exact_b128": lambda i: dt.build_tree_sequential(r1["draft"], E, head_d, 1024, 64, r1["root"], 8,
                                                                    128, 0.0, ws=w1["q"], out=tq1),
        "gated": lambda i: dt.build_tree_gated(r1["talon"], 10, 0.03, 60, ws=w1["g"], out=tg1),
        "static_k10_d6": lambda i: dt.build_tree_static(r1["talon"], 10, 6, ws=w1["s"], out=ts1),
        "tdes_k32_b128": lambda i: dt.build_tree_tdes(r1["draft"], r1["root_g"], mlp, 32, 128, ws=w1["e"], out=tt1),
        "accept_t0": lambda i: dt.accept_tree(tm_1, r1["target"], None, 0.0, synth.PHILOX_SEED, i, 1, ws=w1["a"],
                                              outs=o1r),
        "accept_t1": lambda i: dt.accept_tree(tm_1, r1["target"], r1["draft"], 1.0, synth.PHILOX_SEED, i, 1,
                                              ws=w1["a"], outs=o1r),
        "accept_match_t1": lambda i: dt.accept_tree_match(tm_1, r1["target"], 1.0, synth.PHILOX_SEED, i, 1,
                                                          ws=w1["a"], outs=o1r),
    }
    r1_us = {}
    for name, fn in ops1.items():
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            fn(i)
            b.record(stream)
        torch.cuda.synchronize()
        r1_us[name] = round(float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3, 2)

    out = {
        "metric": "tree-build rounds/sec + us/round at V=151936,L=16,B=128; HBM GB/s vs peak",
        "value": round(value, 1), "unit": "rounds/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "us_per_round": round(ms_per_step * 1e3 / R, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "R=64 rounds, L=16, V=151936 bf16: one row sweep (K=64) of the DDTree-shape logits "
                               "shared by marginal K=B=64 and depthwise K=8,W=32,B=128,beta=-0.5,E 151936x1024,rank 64 "
                               "(head prepared once) + gated K_root=10,mu=0.03,N=60 (TALON-shape logits, own sweep) + "
                               "accept T=0 and T=1 (1 trial/round, one workgroup per round) on the marginal trees",
                   "rounds": R, "L": L, "V": V},
        "per_config_ms": {n: round(v, 4) for n, v in per_config.items()},
        "per_config_us_per_round": {n: round(v * 1e3 / R, 3) for n, v in per_config.items()},
        "schedule": "draft row sweep -> marginal (its lists) -> accept_tree_narrow T=1 -> T=0 on one stream, depthwise "
                    "(the same lists) on a second once they are written, gated (own sweep) on a third (default "
                    "priority), forked and joined per step",
        "walk_failures": walk_failures,
        "breakdown_us_per_round": {n: round(float(np.median(per[:, k])) * 1e3 / R, 3) for k, n in enumerate(names)},
        "breakdown_ms": {n: round(float(np.median(per[:, k])), 4) for k, n in enumerate(names)},
        "breakdown_ms_mean": {n: round(float(per[:, k].mean()), 4) for k, n in enumerate(names)},
        "breakdown_calls": n_ser,
        "event_ms_per_step_serial": round(step_ms, 4),
        "roofline": roofline,
        "extra_ms": extra_ms,
        "r1_latency_us": r1_us,
        "correction_gemm": correction_gemm(os.path.join(ROOT, "profiles", "depthwise_corr_counters.json")),
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


_ORACLE = {}


def _oracle_init(U_bits, P_bits):
    """Worker set-up for the oracle leg: one BLAS thread, the head's U and P widened once."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        _ORACLE["limit"] = threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    widen = lambda b: (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _ORACLE["U"], _ORACLE["P"] = widen(U_bits), widen(P_bits)


class _Rows:
    """Rows of E gathered for one round, indexed like the full table."""

    def __init__(self, toks, rows):
        import numpy as np
        self.at = {int(t): i for i, t in enumerate(toks)}
        self.rows = (np.asarray(rows, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)

    def __getitem__(self, idx):
        import numpy as np
        idx = np.atleast_1d(np.asarray(idx))
        return self.rows[[self.at[int(t)] for t in idx]].astype(np.float64)


def _oracle_round(args):
    """One round of the whole step on the oracle, each operation timed on its own (seconds).
    The round's target rows follow its marginal tree and are drawn untimed."""
    import numpy as np
    import synth
    from oracle import accept, depthwise, gated, marginal, rowsweep
    r, draft_r, talon_r, toks, erows, root_r = args
    z = rowsweep.as_f64(draft_r, "bf16")
    tal = rowsweep.as_f64(talon_r, "bf16")
    out = {}
    t0 = time.perf_counter()
    tm = marginal.build_marginal(z, 64, 64, 0.0)
    out["cfg2_marginal"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    depthwise.build_depthwise(z, _Rows(toks, erows), _ORACLE["U"], _ORACLE["P"], int(root_r), 8, 32, 128, -0.5)
    out["cfg3_depthwise"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    gated.build_gated(tal, 10, float(np.float32(0.03)), 60, full_pool=False)
    out["cfg4_gated"] = time.perf_counter() - t0
    depth = np.array(tm.arrays(64)[2])[None, :]
    tgt = rowsweep.as_f64(synth.verification_target(draft_r[None], depth, seed=5)[0], "bf16")
    t0 = time.perf_counter()
    accept.walk_greedy(tm.parent, tm.token, tm.depth, tgt[:tm.n + 1])
    out["cfg5_accept_t0"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    tab = accept.ResidualTables(tm.parent, tm.token, tm.depth, tgt[:tm.n + 1], z, 1.0)
    accept.walk_sampled(tab, tm.depth, synth.PHILOX_SEED, 0, r)
    out["cfg5_accept_t1"] = time.perf_counter() - t0
    return out


def cpu_baseline(draft_h, talon_h, head, n_single=3, n_par=32):
    """The oracle, as it stands, on a bounded sample of the same step: (1) n_single rounds one
    after another in this process on one thread, each operation timed (ms per round per
    config, and the tiny marginal config); (2) the first n_par rounds spread over
    min(16, cpu count) worker processes, one round per task, one thread each: value = rounds
    per second of the whole step, wall clock. float64 numpy throughout."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np
    import synth
    from oracle import marginal, rowsweep

    E_h, U_h, P_h, root_h = head

    def task(r):
        z = rowsweep.as_f64(draft_h[r], "bf16")
        toks = {int(root_h[r])}
        for d in range(z.shape[0]):
            kth = np.partition(z[d], -8)[-8]
            toks.update(int(t) for t in np.nonzero(z[d] >= kth)[0])
        toks = sorted(toks)
        return (r, draft_h[r], talon_h[r], toks, E_h[toks], int(root_h[r]))

    # (1) one thread, rounds in sequence
    _oracle_init(U_h, P_h)
    single = [_oracle_round(task(r)) for r in range(n_single)]
    per_cfg = {k: round(1e3 * float(np.mean([x[k] for x in single])), 2) for k in single[0]}
    tiny = synth.tiny_marginal()
    t0 = time.perf_counter()
    for r in range(tiny.shape[0]):
        marginal.build_marginal(rowsweep.as_f64(tiny[r], "f32"), 8, 8, 0.0)
    per_cfg["cfg1_tiny_marginal"] = round(1e3 * (time.perf_counter() - t0) / tiny.shape[0], 3)
    step_1core = sum(float(np.mean([x[k] for x in single])) for k in single[0])
    _ORACLE.clear()
    # (2) rounds in parallel
    workers = max(1, min(16, os.cpu_count() or 1))
    tasks = [task(r) for r in range(n_par)]
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"), initializer=_oracle_init,
                                initargs=(U_h, P_h)) as pool:
        list(pool.map(_oracle_round, tasks[:workers]))  # start-up and first imports, untimed
        t0 = time.perf_counter()
        list(pool.map(_oracle_round, tasks, chunksize=1))
        wall = time.perf_counter() - t0
    return {"value": round(n_par / wall, 4), "unit": "rounds/s", "cores": workers, "kind": "oracle",
            "sample": f"rounds 0..{n_par - 1} of the full step (marginal + depthwise + gated + accept T=0 + T=1 per "
                      f"round), one round per task over {workers} worker processes of one thread each, float64 "
                      f"numpy; {wall:.2f} s wall",
            "single_thread": {"rounds_per_s": round(1.0 / step_1core, 4), "cores": 1,
                              "ms_per_round": per_cfg,
                              "sample": f"rounds 0..{n_single - 1} in sequence, one thread; cfg1 over its 4 rounds"}}


if __name__ == "__main__":
    main()
