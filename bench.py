#!/usr/bin/env python3
"""MoE decode benchmark on one MI355X: 60 HBM-resident layers x 512 4-bit
experts (plus a shared expert and a bf16 router per layer), batch 1.

A step is one decode token: 60 sequential moe_layer_decode calls (router,
softmax/top-4/renormalise, dequantised gate/up/down GEMVs of 4 routed experts
plus the shared expert, SwiGLU, weighted combine), replayed from a hipGraph
captured per token.  Inputs are synthetic (seeded) and resident in HBM before
the timed region starts; consecutive tokens are AR(1)-correlated so that about
70% of the routed experts repeat from one token to the next.

Prints one JSON line (see the repository's design notes for every field).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128, help="timed decode tokens")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="stack60", choices=["stack60", "stack60_chain", "stack60_2bit", "layer",
                                                         "batch64", "prefill4096", "stack8_tier"])
    ap.add_argument("--layers", type=int, default=None, help="override layer count (testing)")
    ap.add_argument("--tokens", type=int, default=None, help="override distinct tokens")
    ap.add_argument("--cpu-layers", type=int, default=20,
                    help="layers of the one-core CPU oracle sample (token 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--check-layers", type=int, default=60,
                    help="layers of token 0 checked against the oracle (the parity gate)")
    ap.add_argument("--reps", type=int, default=5,
                    help="repetitions of the timed region for the spread")
    ap.add_argument("--per-layer", action="store_true",
                    help="one moe_layer_decode call per layer instead of one multi-layer call "
                         "per token")
    ap.add_argument("--compare-paths", type=int, default=1,
                    help="also time the other path on a few tokens (0: skip)")
    ap.add_argument("--timing", action="store_true",
                    help="after the timed region, a per-stage breakdown of a few eager steps "
                         "(moe_timing_*; the stack workloads: the multi-layer and the per-layer "
                         "path) in the JSON line's \"stages\"")
    ap.add_argument("--layer-trace", action="store_true",
                    help="after the timed region, one token's per-layer step times from the "
                         "multi-layer kernel's own timestamps (needs a library built with "
                         "-DMOE_STACK_TRACE, loaded through MOE_LIB) in the JSON line's "
                         "\"layer_trace\"")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (calibrates the HBM "
                         "byte counters of the profiler) and exit")
    return ap.parse_args()


KERNEL_SOURCES = ["bit_dequant_expert_moe_amd/csrc/moe_fused.hip",
                  "bit_dequant_expert_moe_amd/csrc/moe_stack.hip",
                  "bit_dequant_expert_moe_amd/csrc/moe_fused_dev.h",
                  "bit_dequant_expert_moe_amd/csrc/moe_device.h",
                  "bit_dequant_expert_moe_amd/csrc/moe_internal.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch from the committed profiler counter summary
    profiles/<name>_hbm_counters.txt (FETCH_SIZE and WRITE_SIZE, each scaled by
    what the counter reads for a plain copy of known size).  None when the
    summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", name + "_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("kernel_source_sha256") == kernel_source_hash():
                return rec
    return None


def calib_copy(mb):
    """A plain copy kernel of known size: reads and writes mb * 2^20 bytes per
    launch, so FETCH_SIZE / WRITE_SIZE of the profiler can be scaled to bytes."""
    import torch
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 4}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        return calib_copy(args.calib_copy)
    import torch
    import bit_dequant_expert_moe_amd as moe
    import synth
    from synth.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    if wl.name == "layer":
        return bench_layer(args, wl)
    if wl.T > 1:
        return bench_batch(args, wl)
    if wl.tier_slots:
        return bench_tier(args, wl)
    nl = args.layers or wl.layers
    ntok = args.tokens or wl.tokens
    dims = moe.Dims(hidden=wl.H, inter=wl.I, n_experts=wl.E, top_k=wl.K, bits=wl.bits,
                    has_shared=wl.has_shared)
    blob = moe.moe_expert_bytes(dims)
    stride = blob
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    params = synth.BlobParams(seed=wl.blob_seed, H=wl.H, I=wl.I, bits=wl.bits, z_lo=wl.z_lo,
                              z_hi=wl.z_hi)
    SHARED_ID = 0xFFFF

    # ---- resident inputs ---------------------------------------------------
    t0 = time.time()
    experts, shared, routers, layers_c = [], [], [], []
    routers_h = []
    for l in range(nl):
        ex = torch.empty(wl.E * stride, dtype=torch.uint8, device=dev)
        synth.gen_blobs_dev(params, l, 0, wl.E, ex.data_ptr(), stride, sp)
        sh = torch.empty(blob, dtype=torch.uint8, device=dev)
        synth.gen_blobs_dev(params, l, SHARED_ID, 1, sh.data_ptr(), blob, sp)
        rh = synth.router_weights(wl.seed, l, wl.E, wl.H)
        routers_h.append(rh)
        r = torch.from_numpy(rh.view(np.int16)).to(dev)
        experts.append(ex)
        shared.append(sh)
        routers.append(r)
        layers_c.append(moe.make_layer(r, ex, stride, sh))
    x_h = np.stack([synth.tokens_ar1(wl.seed, l, ntok, wl.H, wl.rho) for l in range(nl)], axis=1)
    x = torch.from_numpy(x_h.view(np.int16)).to(dev)            # [ntok][nl][H] bf16
    chain = wl.chain
    if chain:
        # the residual stream of each token before layer 0; every layer forms
        # its x from it (written to x[t][l]) and adds its y into it
        r0_h = synth.residual(wl.seed, ntok, wl.H, wl.rho) * np.float32(wl.resid_scale)
        r0 = torch.from_numpy(r0_h).to(dev)                     # [ntok][H] fp32
        r = torch.empty_like(r0)
    y = torch.empty((ntok, nl, wl.H), dtype=torch.float32, device=dev)
    ids = torch.zeros((ntok, nl, wl.K), dtype=torch.int32, device=dev)
    wts = torch.zeros((ntok, nl, wl.K), dtype=torch.float32, device=dev)
    ws_bytes = moe.moe_workspace_bytes(dims, 1)
    ws = moe.alloc_workspace(dims, 1)
    torch.cuda.synchronize()
    log("resident: %d layers x %d experts (%.1f GB) in %.1fs" % (
        nl, wl.E, nl * (wl.E + 1) * blob / 1e9, time.time() - t0))

    layer_arr = moe.layer_array(layers_c)
    stack_path = not args.per_layer

    def call_layer(t, l, sp_):
        if chain:
            moe.moe_layer_decode_residual(dims, layers_c[l], r[t], 1, x[t, l], y[t, l],
                                          ids[t, l], wts[t, l], ws, ws_bytes, sp_)
        else:
            moe.moe_layer_decode(dims, layers_c[l], x[t, l], 1, y[t, l], ids[t, l], wts[t, l],
                                 ws, ws_bytes, sp_)

    def call_token(t, sp_, stack):
        # the token's layers: one multi-layer call, or one call per layer
        if stack:
            if chain:
                moe.moe_stack_decode_residual(dims, layer_arr, r[t], x[t], y[t], ids[t], wts[t],
                                              ws, ws_bytes, sp_)
            else:
                moe.moe_stack_decode(dims, layer_arr, x[t], y[t], ids[t], wts[t], ws, ws_bytes,
                                     sp_)
        else:
            for l in range(nl):
                call_layer(t, l, sp_)

    def enqueue_token(t, sp_, stack=stack_path):
        # on the chain, the token's residual is restored first (a 16 KB device
        # copy on torch's current stream, inside the step)
        if chain:
            r[t].copy_(r0[t])
        call_token(t, sp_, stack)

    def capture(n, stack):
        gs = []
        cs = torch.cuda.Stream()
        with torch.cuda.stream(cs):
            for t in range(n):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    enqueue_token(t, torch.cuda.current_stream().cuda_stream, stack)
                gs.append(g)
        torch.cuda.synchronize()
        return gs

    # ---- one graph per token ------------------------------------------------
    enqueue_token(0, sp)  # eager run first (also checks the path)
    torch.cuda.synchronize()
    graphs = capture(ntok, stack_path)
    log("captured %d token graphs of %d layers (%s)" % (
        ntok, nl, "one multi-layer call" if stack_path else "one call per layer"))

    for i in range(args.warmup):
        graphs[i % ntok].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % ntok].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps
    tok_s = 1000.0 / ms_per_step
    expert_bytes_tok = nl * (wl.K + wl.has_shared) * blob
    router_bytes_tok = nl * wl.E * wl.H * 2
    expert_gbs = expert_bytes_tok * tok_s / 1e9
    all_gbs = (expert_bytes_tok + router_bytes_tok) * tok_s / 1e9
    log("decode: %.3f ms/token, %.1f tok/s, %.0f layers/s, expert GB/s %.0f (%.1f%% of 8 TB/s),"
        " all-bytes GB/s %.0f" % (ms_per_step, tok_s, tok_s * nl, expert_gbs,
                                   100 * expert_gbs / HBM_PEAK_GBS, all_gbs))

    # routing reuse between consecutive tokens (from every token's ids)
    for t in range(ntok):
        graphs[t].replay()
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    reuse = np.mean([len(set(ids_h[t, l]) & set(ids_h[t - 1, l])) / wl.K
                     for t in range(1, ntok) for l in range(nl)]) if ntok > 1 else float("nan")
    log("expert reuse between consecutive tokens: %.3f" % reuse)

    # ---- spread over repetitions of the timed region -------------------------
    rep_tok_s = []
    for _ in range(args.reps):
        e0.record()
        for i in range(args.steps):
            graphs[i % ntok].replay()
        e1.record()
        torch.cuda.synchronize()
        rep_tok_s.append(1000.0 * args.steps / e0.elapsed_time(e1))
    reps = spread(rep_tok_s)
    log("tok/s over %d repetitions: median %.1f, p10 %.1f, p90 %.1f" % (
        args.reps, reps["median"], reps["p10"], reps["p90"]))

    # ---- per-launch duration of the dominant kernel ------------------------------
    # Multi-layer path: a token graph is one k_stack launch (plus, on the chain,
    # the 16 KB restore of the token's residual); per-layer path: nl k_layer1
    # launches back to back.  The timed region above (HIP events on the replay
    # stream) divided by the launches it holds is the average launch duration.
    # Launches between their own events are reported beside it (the events add
    # a gap per launch).
    fused = os.environ.get("MOE_DISABLE_FUSED", "0") != "1"
    layer_bytes = router_bytes_tok // nl + (wl.K + wl.has_shared) * blob
    layer_us = ms_per_step * 1e3 / nl
    t_tok = 1 % ntok
    if stack_path:
        launch_us = ms_per_step * 1e3
        launch_bytes = nl * layer_bytes
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(8)]
        for i in range(8):
            ev[i][0].record()
            call_token((t_tok + i) % ntok, sp, True)
            ev[i][1].record()
        torch.cuda.synchronize()
        iso_us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
        kname = "k_stack_%s" % wl.name
    else:
        launch_us = layer_us
        launch_bytes = layer_bytes
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(nl)]
        torch.cuda._sleep(100_000_000)
        for l in range(nl):
            ev[l][0].record()
            call_layer(t_tok, l, sp)
            ev[l][1].record()
        torch.cuda.synchronize()
        iso_us = float(np.mean([ev[l][0].elapsed_time(ev[l][1]) * 1e3 for l in range(nl)]))
        kname = "k_layer1_%s" % wl.name
    achieved = launch_bytes / (launch_us * 1e-6) / 1e9
    log("%s: %.2f us per launch in the token graphs (%.2f us between events), %.2f us per "
        "layer -> %.0f GB/s of algorithmic bytes (%d B per launch)" % (
            "k_stack" if stack_path else "k_layer1", launch_us, iso_us, layer_us, achieved,
            launch_bytes))
    traffic = measured_traffic(kname) if fused else None
    err = moe.moe_get_device_error(ws, sp)
    if err:
        log("device error flags: %d" % err)

    # ---- the other path, for comparison (a few tokens) -------------------------
    other = None
    if fused and args.compare_paths:
        nt = min(16, ntok)
        g2 = capture(nt, not stack_path)
        for i in range(4):
            g2[i % nt].replay()
        e0.record()
        for i in range(4 * nt):
            g2[i % nt].replay()
        e1.record()
        torch.cuda.synchronize()
        o_ms = e0.elapsed_time(e1) / (4 * nt)
        other = {"path": "one call per layer" if stack_path else "one multi-layer call",
                 "tokens_per_s": 1000.0 / o_ms, "us_per_layer": o_ms * 1e3 / nl}
        del g2
        log("the other path (%s): %.1f tok/s, %.2f us per layer" % (
            other["path"], other["tokens_per_s"], other["us_per_layer"]))
        graphs[0].replay()
        torch.cuda.synchronize()

    # ---- measured streaming-read rate at the layer's and the token's size -----
    stream = stream_read_rates(torch, moe, experts, layer_bytes, nl * layer_bytes, sp)
    stream["layer_frac_of_layer_size_rate"] = (layer_bytes / (layer_us * 1e-6) / 1e9 /
                                               stream["layer_size_back_to_back_GBps"])
    stream["token_frac_of_token_size_rate"] = (
        (expert_bytes_tok + router_bytes_tok) * tok_s / 1e9 / stream["token_size_single_launch_GBps"])
    log("stream read: %.0f GB/s per launch of %d B back to back (%.0f GB/s isolated), "
        "%.0f GB/s for one launch of %d B" % (
            stream["layer_size_back_to_back_GBps"], launch_bytes,
            stream["layer_size_isolated_GBps"], stream["token_size_single_launch_GBps"],
            stream["token_bytes"]))

    # ---- parity gate: every layer of token 0 against the float64 oracle -----
    import oracle
    oracle.set_threads(os.cpu_count() or 1)
    od = oracle.Dims(H=wl.H, I=wl.I, E=wl.E, K=wl.K, bits=wl.bits, has_shared=wl.has_shared)
    graphs[0].replay()
    torch.cuda.synchronize()
    check = parity_check(oracle, od, wl, nl, args.check_layers, x, y, ids, wts, experts, shared,
                         routers_h, x_h, r0_h if chain else None, stride, blob, chain)

    # ---- CPU baseline: the float64 oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(oracle, od, wl, nl, args.cpu_layers, experts, shared, routers_h, x_h,
                           r0_h if chain else None, stride, blob, chain)

    out = {
        "metric": "MoE decode tokens/s (60 layers, batch 1) + expert-weight GB/s as % HBM peak",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u%d" % wl.bits + "+bf16/fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": nl, "experts": wl.E, "top_k": wl.K,
                   "shared_experts": wl.has_shared, "hidden": wl.H, "inter": wl.I,
                   "bits": wl.bits, "group": 64, "batch": 1, "tokens": ntok,
                   "expert_reuse": reuse},
        "expert_weight_GBps": expert_gbs,
        "expert_weight_frac_hbm_peak": expert_gbs / HBM_PEAK_GBS,
        "all_bytes_GBps": all_gbs,
        "layers_per_s": tok_s * nl,
        "repetitions": dict(reps, unit="tokens/s", n=args.reps, steps_each=args.steps),
        "roofline": {"bound": "hbm",
                     "kernel": (("k_stack (moe_stack_decode_residual)" if chain else
                                 "k_stack (moe_stack_decode)") if stack_path else
                                ("k_layer1 (moe_layer_decode_residual)" if chain else
                                 "k_layer1 (moe_layer_decode)")) if fused else
                               "moe_layer_decode (k_route + k_gateup + k_down)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
                     "avg_launch_us": launch_us, "between_events_launch_us": iso_us,
                     "bytes_per_launch": launch_bytes, "us_per_layer": layer_us,
                     "layers_per_launch": nl if stack_path else 1},
        "other_path": other,
        "stream_read": stream,
        "device_error_flags": err,
        "parity": check,
        "parity_ok": check["ok"],
        "cpu_baseline": cpu,
    }
    if args.layer_trace and stack_path and fused:
        tr = layer_trace(torch, ws, nl, lambda: enqueue_token(0, sp, True))
        if tr is None:
            log("layer trace: the library was built without MOE_STACK_TRACE")
        else:
            for name, v in tr["steps"].items():
                log("  %-26s median %6.2f  p90 %6.2f us" % (name, v["median_us"], v["p90_us"]))
            log("  layer period %.2f us, logits polls per layer %.1f" % (
                tr["layer_period_us"], tr["logits_polls_per_layer"]))
        out["layer_trace"] = tr
    if args.timing:
        out["stages"] = {}
        for name, stk in (("multi-layer", True), ("per-layer", False)):
            if stk and not fused:
                continue
            st = stage_breakdown(torch, moe, lambda i, stk=stk: enqueue_token(i % ntok, sp, stk), 4)
            log_stages(name, st)
            out["stages"][name] = st
    print(json.dumps(out), flush=True)
    if not check["ok"] or err:
        log("PARITY FAILED (or device error): see the parity object")
        sys.exit(3)


def stage_breakdown(torch, moe, step, n):
    """Per-stage times of n eager steps (HIP events the library records while
    moe_timing is on), microseconds and calls per step.  Outside the timed
    region: the events add host work to every stage."""
    torch.cuda.synchronize()
    moe.moe_timing_set(True)
    try:
        moe.moe_timing_read(reset=True)
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        t = moe.moe_timing_read(reset=True)
    finally:
        moe.moe_timing_set(False)
    return {k: {"us_per_step": ms * 1e3 / n, "calls_per_step": c / n} for k, (ms, c) in t.items()}


def log_stages(name, st):
    log("stages (%s): %s" % (name, ", ".join("%s %.1f us x %.0f" % (k, v["us_per_step"],
                                                                   v["calls_per_step"])
                                             for k, v in st.items())))


# Steps the multi-layer kernel timestamps in a build with MOE_STACK_TRACE
# (event number -> name); event 26 holds the logits poll count x 100.
TRACE_EVENTS = {
    15: "r gathered", 27: "gate/up: r read", 28: "gate/up: norm done",
    30: "gate/up: x from LDS", 31: "gate/up: router partials", 29: "gate/up: staged",
    0: "A (exchange)", 8: "A (gate/up)", 1: "logits published", 25: "first logits poll issued",
    5: "first logits poll back", 34: "logits taken", 32: "top-K selected",
    9: "shared gate/up published", 2: "top-K done", 6: "first shared h poll back",
    10: "routed loads issued", 19: "row: routed loads issued", 3: "shared h read",
    20: "row: shared rows done", 11: "slot 0 published", 16: "slot 0 h read",
    21: "row: slot 0 rows done", 12: "slot 1 published", 17: "slot 1 h read",
    22: "row: slot 1 rows done", 13: "slot 2 published", 18: "slot 2 h read",
    23: "row: slot 2 rows done", 14: "slot 3 published", 4: "slot 3 h read",
    24: "row: slot 3 rows done", 7: "layer end (y)"}


def layer_trace(torch, ws, nl, run):
    """One token's per-layer step times from the multi-layer kernel's
    timestamps.  The trace buffer's device address goes into the workspace's
    control block (bytes 8..15) for one call and is cleared after it.  Per
    step: median and 90th percentile over workgroups and the inner layers of
    the time since the layer's first barrier (earliest workgroup), in us; the
    device clock counts at 100 MHz.  None when the library was built without
    the timestamps."""
    nev, maxl, nwg = 48, 64, 256
    buf = torch.zeros(nwg * maxl * nev, dtype=torch.int64, device=ws.device)
    torch.cuda.synchronize()
    ws[8:16].copy_(torch.tensor([buf.data_ptr()], dtype=torch.int64).view(torch.uint8))
    try:
        run()
        torch.cuda.synchronize()
    finally:
        ws[8:16].zero_()
        torch.cuda.synchronize()
    T = buf.cpu().numpy().reshape(nwg, maxl, nev)[:, :nl, :].astype(np.float64) * 0.01
    if not T.any() or nl < 3:
        return None
    R = np.stack([np.where(T[:, l, :] > 0, T[:, l, :] - T[:, l, 0].min(), np.nan)
                  for l in range(1, nl - 1)])
    steps = {}
    for ev, name in TRACE_EVENTS.items():
        v = R[:, :, ev]
        if np.all(np.isnan(v)):
            continue
        steps[name] = {"median_us": float(np.nanmedian(v)), "p90_us": float(np.nanpercentile(v, 90))}
    starts = np.array([T[:, l, 0].min() for l in range(nl)])
    return {"steps": dict(sorted(steps.items(), key=lambda kv: kv[1]["median_us"])),
            "layer_period_us": float(np.median(np.diff(starts))),
            "logits_polls_per_layer": float(np.median(T[:, 1:nl - 1, 26]))}


def host_cores():
    """Threads for the oracle: the cores this process may run on, capped by
    OMP_NUM_THREADS when it is set (the count may exceed the host's share
    otherwise)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def spread(vals):
    v = np.asarray(vals, dtype=np.float64)
    return {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
            "p90": float(np.percentile(v, 90)), "min": float(v.min()), "max": float(v.max())}


def stream_read_rates(torch, moe, buffers, layer_bytes, token_bytes, sp):
    """moe_stream_read over resident expert memory that the decode did not
    just touch: one launch per buffer of layer_bytes (back to back, and each
    between its own events), and one launch of token_bytes (capped at a
    buffer's size)."""
    n = len(buffers)
    off = (buffers[0].numel() // 3) // 256 * 256
    lb = layer_bytes // 16 * 16
    tb = min(token_bytes, buffers[0].numel() - 256) // 16 * 16
    sink = torch.empty(moe.moe_stream_read_sink_words(max(lb, tb)), dtype=torch.int32,
                       device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    moe.moe_flush(flush, flush.numel(), sp)
    e0.record()
    for i in range(n):
        moe.moe_stream_read(buffers[i][off:], lb, sink, sp)
    e1.record()
    torch.cuda.synchronize()
    b2b_us = e0.elapsed_time(e1) * 1e3 / n
    iso = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    moe.moe_flush(flush, flush.numel(), sp)
    for i in range(n):
        evs[i][0].record()
        moe.moe_stream_read(buffers[(i + n // 2) % n][off + lb:], lb, sink, sp)
        evs[i][1].record()
    torch.cuda.synchronize()
    iso = [a.elapsed_time(b) * 1e3 for a, b in evs]
    tok_us = []
    for i in range(3):
        moe.moe_flush(flush, flush.numel(), sp)
        e0.record()
        moe.moe_stream_read(buffers[i % n], tb, sink, sp)
        e1.record()
        torch.cuda.synchronize()
        tok_us.append(e0.elapsed_time(e1) * 1e3)
    return {"layer_bytes": lb, "layer_size_back_to_back_us": b2b_us,
            "layer_size_back_to_back_GBps": lb / b2b_us / 1e3,
            "layer_size_isolated_us": float(np.median(iso)),
            "layer_size_isolated_GBps": lb / float(np.median(iso)) / 1e3,
            "token_bytes": tb, "token_size_single_launch_us": float(np.median(tok_us)),
            "token_size_single_launch_GBps": tb / float(np.median(tok_us)) / 1e3}


def parity_check(oracle, od, wl, nl, n_check, x, y, ids, wts, experts, shared, routers_h, x_h,
                 r0_h, stride, blob, chain):
    """Token 0 of the last replay, layer by layer, against the float64 oracle:
    ids exact where the float64 gap is at least 1e-3 (else each pick within
    1e-3 of the correct logit at its rank), w within 1e-5 of the float64
    softmax of the pick, y within 2e-3 max|y| teacher-forced on the x and
    the pick the GPU used; on the chain also the x each layer formed against
    the oracle's norm of the residual (rebuilt as r + y in fp32)."""
    TIE, WT, YT = 1e-3, 1e-5, 2e-3
    xk = x[0].cpu().numpy().view(np.uint16) if chain else x_h[0]
    yk, idk, wk = y[0].cpu().numpy(), ids[0].cpu().numpy(), wts[0].cpu().numpy()
    rr = r0_h[0].copy() if chain else None
    worst, worst_w, bad, norm_mis, near_ties = 0.0, 0.0, [], 0, 0
    n_check = min(n_check, nl)
    for l in range(n_check):
        if chain:
            xo = oracle.rmsnorm_bf16(rr)
            d = xk[l].astype(np.int32) - xo.astype(np.int32)
            nm = int(np.count_nonzero(d))
            norm_mis += nm
            if nm > 8 or np.any(np.abs(d) > 1):
                bad.append("layer %d: x differs from the oracle's norm in %d elements" % (l, nm))
            rr = (rr + yk[l]).astype(np.float32)
        _, _, lg, gap = oracle.route(od, routers_h[l], xk[l][None])
        lg, gap = lg[0], float(gap[0])
        order = np.lexsort((np.arange(lg.size), -lg))[:wl.K]
        if gap >= TIE:
            if not np.array_equal(idk[l], order):
                bad.append("layer %d: ids %s, oracle %s" % (l, idk[l].tolist(), order.tolist()))
        else:
            near_ties += 1
            if np.any(np.abs(lg[idk[l]] - lg[order]) > TIE) or len(set(idk[l].tolist())) != wl.K:
                bad.append("layer %d: ids %s not within the near-tie margin" % (
                    l, idk[l].tolist()))
        sel = lg[idk[l]]
        wo = np.exp(sel - sel.max())
        wo /= wo.sum()
        worst_w = max(worst_w, float(np.max(np.abs(wk[l] - wo))))
        if abs(float(np.sum(wk[l], dtype=np.float64)) - 1) > 1e-6 or np.max(np.abs(wk[l] - wo)) > WT:
            bad.append("layer %d: w %s, oracle %s" % (l, wk[l].tolist(), wo.tolist()))
        blobs = {int(e): experts[l][int(e) * stride:int(e) * stride + blob].cpu().numpy()
                 for e in idk[l]}
        yo = oracle.expert_forward(od, blobs, shared[l].cpu().numpy(), xk[l][None], idk[l][None],
                                   wo[None])[0]
        e_l = float(np.max(np.abs(yk[l] - yo)) / np.max(np.abs(yo)))
        worst = max(worst, e_l)
        if not e_l <= YT:
            bad.append("layer %d: max|dy|/max|y| = %.2e" % (l, e_l))
    ok = not bad
    log("oracle check of token 0, %d layers: max|dy|/max|y| = %.2e, max|dw| = %.1e, %d near "
        "ties, %s" % (n_check, worst, worst_w, near_ties, "ok" if ok else "FAILED"))
    for b in bad:
        log("  " + b)
    out = {"ok": ok, "token": 0, "layers_checked": n_check, "max_rel_err_y": worst,
           "max_abs_err_w": worst_w, "near_ties": near_ties, "y_tol": YT, "failures": bad[:10]}
    if chain:
        out["x_norm_mismatches"] = norm_mis
    return out


def cpu_baseline(oracle, od, wl, nl, n_single, experts, shared, routers_h, x_h, r0_h, stride,
                 blob, chain):
    """The float64 oracle on token 0 of the workload: every layer on all host
    cores (output rows over threads, results independent of the count), and
    the first n_single layers on one core, timed without the device-to-host
    copies of the selected experts."""
    data = []
    rr = r0_h[0:1] if chain else None
    fetch = lambda l: (lambda e: experts[l][e * stride:e * stride + blob].cpu().numpy())
    oracle.set_threads(1)
    for l in range(nl):
        if chain:
            xo = oracle.rmsnorm_bf16(rr)
        else:
            xo = x_h[0, l][None]
        ido, _, _, _ = oracle.route(od, routers_h[l], xo)
        blobs = {int(e): fetch(l)(int(e)) for e in ido[0]}
        data.append((blobs, shared[l].cpu().numpy()))
        if chain:
            rr = oracle.residual_layer(od, routers_h[l], blobs, data[l][1], rr)[0].astype(np.float32)

    def run(n):
        rr = r0_h[0:1] if chain else None
        tc = time.perf_counter()
        for l in range(n):
            if chain:
                rr = oracle.residual_layer(od, routers_h[l], data[l][0], data[l][1],
                                           rr)[0].astype(np.float32)
            else:
                oracle.layer(od, routers_h[l], data[l][0], data[l][1], x_h[0, l][None])
        return time.perf_counter() - tc

    ns = max(1, min(n_single, nl))
    oracle.set_threads(1)
    dt1 = run(ns)
    cores = host_cores()
    oracle.set_threads(cores)
    dta = run(nl)
    oracle.set_threads(1)
    tok1, toka = 1.0 / (dt1 * nl / ns), 1.0 / dta
    log("cpu oracle: 1 core %.1f s for %d layers -> %.4f tok/s; %d threads %.1f s for %d layers "
        "-> %.4f tok/s" % (dt1, ns, tok1, cores, dta, nl, toka))
    return {"value": toka, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "token 0, all %d layers, output rows over %d threads (%.1f s)" % (
                nl, cores, dta),
            "single_core": {"value": tok1, "unit": "tokens/s", "cores": 1,
                            "sample": "token 0, layers 0..%d of %d (%.1f s), scaled to %d layers"
                                      % (ns - 1, nl, dt1, nl)}}


def bench_layer(args, wl):
    """One full 512-expert layer, one token per call, with the last-level cache
    flushed (512 MB of stores, then 512 MB of reads of other memory) before
    every call: the call's events exclude the flush.  128 distinct tokens (independent activations, so distinct
    routings), cycled.  value = calls per second from the summed call times."""
    import torch
    import bit_dequant_expert_moe_amd as moe
    import synth
    import oracle
    dims = moe.Dims(hidden=wl.H, inter=wl.I, n_experts=wl.E, top_k=wl.K, bits=wl.bits,
                    has_shared=wl.has_shared)
    blob = moe.moe_expert_bytes(dims)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sp = torch.cuda.current_stream().cuda_stream
    params = synth.BlobParams(seed=wl.blob_seed, H=wl.H, I=wl.I, bits=wl.bits)
    ex = torch.empty(wl.E * blob, dtype=torch.uint8, device=dev)
    synth.gen_blobs_dev(params, 0, 0, wl.E, ex.data_ptr(), blob, sp)
    sh = torch.empty(blob, dtype=torch.uint8, device=dev)
    synth.gen_blobs_dev(params, 0, 0xFFFF, 1, sh.data_ptr(), blob, sp)
    rh = synth.router_weights(wl.seed, 0, wl.E, wl.H)
    r = torch.from_numpy(rh.view(np.int16)).to(dev)
    L = moe.make_layer(r, ex, blob, sh)
    ntok = args.tokens or wl.tokens
    x_h = synth.tokens(wl.seed, 0, ntok, wl.H)
    x = torch.from_numpy(x_h.view(np.int16)).to(dev)
    y = torch.empty((ntok, wl.H), dtype=torch.float32, device=dev)
    ids = torch.empty((ntok, wl.K), dtype=torch.int32, device=dev)
    wts = torch.empty((ntok, wl.K), dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(dims, 1)
    wsb = ws.numel()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    clean = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    clean.fill_(7)
    sink = torch.empty(moe.moe_stream_read_sink_words(clean.numel()), dtype=torch.int32,
                       device=dev)

    def call(t):
        moe.moe_layer_decode(dims, L, x[t], 1, y[t], ids[t], wts[t], ws, wsb, sp)

    def flush_caches():
        # 512 MB of stores, then a 512 MB read of other memory, so that the
        # cache holds clean unrelated lines (no write-back of the flush's own
        # lines inside the timed call)
        moe.moe_flush(flush, flush.numel(), sp)
        moe.moe_stream_read(clean, clean.numel(), sink, sp)

    for i in range(args.warmup):
        flush_caches()
        call(i % ntok)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        flush_caches()
        evs[i][0].record()
        call(i % ntok)
        evs[i][1].record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    err = moe.moe_get_device_error(ws, sp)
    layer_bytes = wl.E * wl.H * 2 + (wl.K + wl.has_shared) * blob
    value = len(us) / (us.sum() * 1e-6)
    achieved = layer_bytes / (np.mean(us) * 1e-6) / 1e9
    sp_us = spread(us)
    log("layer call with flushed caches: median %.2f us (p10 %.2f, p90 %.2f), %.0f layers/s, "
        "%.0f GB/s of algorithmic bytes (%.1f%% of 8 TB/s)" % (
            sp_us["median"], sp_us["p10"], sp_us["p90"], value, achieved,
            100 * achieved / HBM_PEAK_GBS))
    # parity gate: the first tokens against the oracle, teacher-forced
    oracle.set_threads(os.cpu_count() or 1)
    od = oracle.Dims(H=wl.H, I=wl.I, E=wl.E, K=wl.K, bits=wl.bits, has_shared=wl.has_shared)
    fetch = lambda e: ex[e * blob:(e + 1) * blob].cpu().numpy()
    n_chk = min(args.check_layers, ntok, 8)
    idh, wh, yh = ids.cpu().numpy(), wts.cpu().numpy(), y.cpu().numpy()
    bad, worst = [], 0.0
    _, _, lg, gap = oracle.route(od, rh, x_h[:n_chk])
    for t in range(n_chk):
        order = np.lexsort((np.arange(wl.E), -lg[t]))[:wl.K]
        if gap[t] >= 1e-3 and not np.array_equal(order, idh[t]):
            bad.append("token %d: ids %s, oracle %s" % (t, idh[t].tolist(), order.tolist()))
        sel = lg[t][idh[t]]
        wo = np.exp(sel - sel.max())
        wo /= wo.sum()
        if np.max(np.abs(wo - wh[t])) > 1e-5:
            bad.append("token %d: w" % t)
        yo = oracle.expert_forward(od, fetch, sh.cpu().numpy(), x_h[t:t + 1], idh[t:t + 1],
                                   wo[None])[0]
        e = float(np.max(np.abs(yh[t] - yo)) / np.max(np.abs(yo)))
        worst = max(worst, e)
        if not e <= 2e-3:
            bad.append("token %d: max|dy|/max|y| = %.2e" % (t, e))
    check = {"ok": not bad, "tokens_checked": n_chk, "max_rel_err_y": worst, "failures": bad}
    log("oracle check of %d tokens: max|dy|/max|y| = %.2e, %s" % (n_chk, worst,
                                                                   "ok" if not bad else bad))
    cpu = None
    if not args.no_cpu_baseline:
        nt = 5
        ido, _, _, _ = oracle.route(od, rh, x_h[:nt])
        blobs = {int(e): fetch(int(e)) for e in np.unique(ido)}
        shh = sh.cpu().numpy()
        cores = host_cores()
        oracle.set_threads(cores)
        tc = time.perf_counter()
        oracle.layer(od, rh, blobs, shh, x_h[:nt])
        dta = time.perf_counter() - tc
        oracle.set_threads(1)
        tc = time.perf_counter()
        oracle.layer(od, rh, blobs, shh, x_h[:1])
        dt1 = time.perf_counter() - tc
        cpu = {"value": nt / dta, "unit": "layers/s", "cores": cores, "kind": "oracle",
               "sample": "%d tokens of the layer, output rows over %d threads (%.1f s)" % (
                   nt, cores, dta),
               "single_core": {"value": 1 / dt1, "unit": "layers/s", "cores": 1,
                               "sample": "1 token of the layer (%.1f s)" % dt1}}
        log("cpu oracle: %.2f layers/s on %d threads, %.2f on one core" % (nt / dta, cores,
                                                                            1 / dt1))
    out = {
        "metric": "MoE layer decode (1 token, one full 512-expert layer, caches flushed): "
                  "layers/s + algorithmic GB/s as % HBM peak",
        "value": value, "unit": "layers/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": float(np.mean(us)) * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u%d+bf16/fp32" % wl.bits, "data": "synthetic",
        "config": {"workload": wl.name, "experts": wl.E, "top_k": wl.K, "bits": wl.bits,
                   "hidden": wl.H, "inter": wl.I, "tokens": ntok, "flush_bytes": flush.numel()},
        "call_us": sp_us,
        "roofline": {"bound": "hbm", "kernel": "moe_layer_decode (k_layer1)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": layer_bytes, "avg_launch_us": float(np.mean(us))},
        "device_error_flags": err, "parity": check, "parity_ok": check["ok"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if bad or err:
        sys.exit(3)


def bench_tier(args, wl):
    """Decode through the off-HBM expert tier: every layer's experts in pinned
    host memory, wl.tier_slots device slots shared by all layers (LRU), router
    and shared expert resident.  A step is one token through all layers
    (moe_tier_decode per layer: route, host waits for the ids, copies of the
    missing experts over PCIe, expert forward).  The cache is warmed with
    `warmup` tokens first.  No graph: the host takes part in every layer."""
    import torch
    import bit_dequant_expert_moe_amd as moe
    import synth
    nl = args.layers or wl.layers
    ntok = args.tokens or wl.tokens
    dims = moe.Dims(hidden=wl.H, inter=wl.I, n_experts=wl.E, top_k=wl.K, bits=wl.bits,
                    has_shared=wl.has_shared)
    blob = moe.moe_expert_bytes(dims)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sp = torch.cuda.current_stream().cuda_stream
    params = synth.BlobParams(seed=wl.blob_seed, H=wl.H, I=wl.I, bits=wl.bits, z_lo=wl.z_lo,
                              z_hi=wl.z_hi)

    def aligned(n, pin=False, device=None):
        t = (torch.empty(n + 256, dtype=torch.uint8, pin_memory=True) if pin else
             torch.empty(n + 256, dtype=torch.uint8, device=device))
        off = (-t.data_ptr()) % 256
        return t[off:off + n]

    t0 = time.time()
    host, shared, routers = [], [], []
    stage = torch.empty(wl.E * blob, dtype=torch.uint8, device=dev)
    for l in range(nl):
        synth.gen_blobs_dev(params, l, 0, wl.E, stage.data_ptr(), blob, sp)
        h = aligned(wl.E * blob, pin=True)
        h.copy_(stage)
        host.append(h)
        sh = torch.empty(blob, dtype=torch.uint8, device=dev)
        synth.gen_blobs_dev(params, l, 0xFFFF, 1, sh.data_ptr(), blob, sp)
        shared.append(sh)
        routers.append(torch.from_numpy(synth.router_weights(wl.seed, l, wl.E, wl.H)
                                        .view(np.int16)).to(dev))
    del stage
    torch.cuda.synchronize()
    log("host tier: %d layers x %d experts (%.1f GB pinned) in %.1fs" % (
        nl, wl.E, nl * wl.E * blob / 1e9, time.time() - t0))
    n_slots = wl.tier_slots
    slots = aligned(n_slots * blob, device=dev)
    staging = aligned(moe.moe_tier_staging_bytes(dims, 1), pin=True)
    scratch = aligned(moe.moe_tier_device_bytes(dims, 1), device=dev)
    copy_stream = torch.cuda.Stream()
    tier = moe.Tier(dims, [h.data_ptr() for h in host], blob, slots, blob, n_slots, staging,
                    scratch, t_max=1, copy_stream=copy_stream)
    wsb = moe.moe_tier_workspace_bytes(dims, n_slots, 1)
    ws = aligned(wsb, device=dev)
    moe.moe_workspace_init(ws, wsb)
    x_h = np.stack([synth.tokens_ar1(wl.seed, l, ntok, wl.H, wl.rho) for l in range(nl)], axis=1)
    x = torch.from_numpy(x_h.view(np.int16)).to(dev)
    y = torch.empty((ntok, nl, wl.H), dtype=torch.float32, device=dev)
    ids = torch.empty((ntok, nl, wl.K), dtype=torch.int32, device=dev)

    def token(t):
        for l in range(nl):
            tier.decode(l, routers[l], shared[l], x[t, l], 1, y[t, l], ids[t, l], None, ws, wsb,
                        sp)

    for i in range(args.warmup):
        token(i % ntok)
    torch.cuda.synchronize()
    st0 = tier.stats()
    tc = time.perf_counter()
    for i in range(args.steps):
        token((args.warmup + i) % ntok)
    torch.cuda.synchronize()
    dt = time.perf_counter() - tc
    st1 = tier.stats()
    hits, misses = st1["hits"] - st0["hits"], st1["misses"] - st0["misses"]
    copied = st1["bytes"] - st0["bytes"]
    ms_per_step = dt * 1e3 / args.steps
    tok_s = args.steps / dt
    hit_rate = hits / max(1, hits + misses)
    log("tier decode: %.3f ms/token (%d layers), %.1f tok/s, %.1f us/layer, hit rate %.3f, "
        "%.2f MB copied per token, %.1f GB/s over PCIe" % (
            ms_per_step, nl, tok_s, ms_per_step * 1e3 / nl, hit_rate, copied / args.steps / 1e6,
            copied / dt / 1e9))
    err = moe.moe_get_device_error(ws, sp)
    out = {
        "metric": "MoE decode tokens/s through the host-memory expert tier (%d layers, batch 1)"
                  % nl,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u%d" % wl.bits + "+bf16/fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": nl, "experts": wl.E, "top_k": wl.K,
                   "bits": wl.bits, "device_slots": n_slots, "tokens": ntok},
        "hit_rate": hit_rate,
        "copied_bytes_per_token": copied / args.steps,
        "pcie_GBps": copied / dt / 1e9,
        "us_per_layer": ms_per_step * 1e3 / nl,
        "device_error_flags": err,
    }
    print(json.dumps(out), flush=True)
    tier.close()


def bench_batch(args, wl):
    """One full layer, T tokens per call routed independently (pairs grouped by
    expert, MFMA GEMMs).  A step is one moe_layer_decode of T tokens; value is
    tokens/s.  Algorithmic bytes per call: router + every distinct selected
    expert once + the shared expert once."""
    import torch
    import bit_dequant_expert_moe_amd as moe
    import synth
    dims = moe.Dims(hidden=wl.H, inter=wl.I, n_experts=wl.E, top_k=wl.K, bits=wl.bits,
                    has_shared=wl.has_shared)
    blob = moe.moe_expert_bytes(dims)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sp = torch.cuda.current_stream().cuda_stream
    params = synth.BlobParams(seed=wl.blob_seed, H=wl.H, I=wl.I, bits=wl.bits)
    ex = torch.empty(wl.E * blob, dtype=torch.uint8, device=dev)
    synth.gen_blobs_dev(params, 0, 0, wl.E, ex.data_ptr(), blob, sp)
    sh = torch.empty(blob, dtype=torch.uint8, device=dev)
    synth.gen_blobs_dev(params, 0, 0xFFFF, 1, sh.data_ptr(), blob, sp)
    rh = synth.router_weights(wl.seed, 0, wl.E, wl.H)
    r = torch.from_numpy(rh.view(np.int16)).to(dev)
    L = moe.make_layer(r, ex, blob, sh)
    nb = 16 if wl.T <= 256 else 4  # distinct batches, cycled
    xs = [torch.from_numpy(synth.tokens(wl.seed, b, wl.T, wl.H).view(np.int16)).to(dev)
          for b in range(nb)]
    y = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
    ids = torch.empty((nb, wl.T, wl.K), dtype=torch.int32, device=dev)
    wts = torch.empty((nb, wl.T, wl.K), dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(dims, wl.T)
    wsb = ws.numel()
    for b in range(nb):
        moe.moe_layer_decode(dims, L, xs[b], wl.T, y, ids[b], wts[b], ws, wsb, sp)
    torch.cuda.synchronize()
    # one graph per batch (route, bucket, x staging, grouped GEMMs, combine)
    graphs = []
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        for b in range(nb):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                moe.moe_layer_decode(dims, L, xs[b], wl.T, y, ids[b], wts[b], ws, wsb,
                                     torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % nb].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % nb].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ids_h = ids.cpu().numpy()
    distinct = float(np.mean([len(np.unique(ids_h[b])) for b in range(nb)]))
    call_bytes = wl.E * wl.H * 2 + (distinct + wl.has_shared) * blob
    gbs = call_bytes / (ms * 1e-3) / 1e9
    tok_s = wl.T / (ms * 1e-3)
    # algorithmic flops: router, and gate, up and down of K + shared slots per token
    flops = 2.0 * wl.T * wl.E * wl.H + 2.0 * wl.T * (wl.K + wl.has_shared) * 3 * wl.H * wl.I
    tflops = flops / (ms * 1e-3) / 1e12
    log("batch of %d tokens: %.1f us per call, %.0f tok/s, %.1f distinct experts, %.0f GB/s "
        "of algorithmic bytes (%.1f%% of 8 TB/s), %.0f TFLOP/s (%.1f%% of bf16 dense peak)" % (
            wl.T, ms * 1e3, tok_s, distinct, gbs, 100 * gbs / HBM_PEAK_GBS, tflops,
            100 * tflops / BF16_PEAK_TFLOPS))
    out = {
        "metric": "MoE layer tokens/s, batch of %d tokens (one 512-expert layer)" % wl.T,
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u%d+bf16/fp32" % wl.bits,
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_call": wl.T, "experts": wl.E,
                   "top_k": wl.K, "bits": wl.bits, "distinct_experts": distinct},
        "roofline": {"bound": "hbm", "kernel": "moe_layer_decode (k_route, k_bucket, "
                     "k_grouped x2, k_combine)", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_call": call_bytes},
        "flops_per_call": flops, "TFLOPs": tflops, "frac_bf16_peak": tflops / BF16_PEAK_TFLOPS,
        "cpu_baseline": None,
    }
    if args.timing:
        st = stage_breakdown(torch, moe, lambda i: moe.moe_layer_decode(
            dims, L, xs[i % nb], wl.T, y, ids[i % nb], wts[i % nb], ws, wsb, sp), 4)
        log_stages("moe_layer_decode", st)
        out["stages"] = st
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
