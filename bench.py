#!/usr/bin/env python3
"""Decode-step throughput of the paged GQA decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b8_bimodal]

One step is the whole hot path over one batch: the host policy and planner
(C++), the hand-over of the task list, the persistent decode kernel and the
merge (fused into the decode kernel, or a second kernel).  The headline batch
is the B=8 bimodal workload (Hq=32, Hkv=8, d=128, page size 16, held-out seed
20260623), drawn in HBM before timing starts; the B=1 long-context workload
(N=32768) is measured the same way in the same run (key "b1").  The K/V pool
is replicated over several "layers" and the steps rotate through them, so
every step streams its KV from HBM rather than from the 256 MB Infinity
Cache, as a model whose layers each own a KV cache does.

Prints one JSON line: decode tokens/s (B tokens per step), KV GB/s, the
roofline of the step's kernels (HIP events on their own dispatches inside the
timed region), the latency of a lone synchronised step (host-planned, and
device-planned replayed from a graph), and the float64 oracle timed on the
host's cores as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "decode tokens/s + achieved KV HBM GB/s (% peak), B8 bimodal Hq32/Hkv8/d128"
HBM_PEAK_GBPS = 8000.0
DEVICE_PLAN_MAX_SPLITS = 64
SPLIT_SWEEP = (8, 16, 32, 64)   # explicit split counts timed on a single-row batch


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(HERE, "paged_gqa_decode_pkv_amd", "csrc", "decode.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload, config):
    """Measured HBM bytes per step from the committed rocprofv3 PMC runs of
    this workload, if they were taken on the current kernel source and on
    this same schedule; else None."""
    try:
        with open(os.path.join(HERE, "profiles", f"decode_{workload}_traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != _kernel_source_hash():
        return None
    if rec.get("config") != config:
        return None
    return rec.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, out_gpu, budget_s: float, rows=None):
    """Time the float64 oracle, as it stands, on the host's cores (its BLAS
    calls may use every core the process may run on), on a bounded sample of
    the same batch: three runs of whole passes, each about budget/3 seconds,
    median reported.  The GPU output on the sample is checked against it."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from workloads import compact_rows

    if rows is None:
        rows = list(range(len(wl.seq_lens_np)))
    q, k, v, bt, sl = compact_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, rows)
    kv_bytes = int(np.asarray(sl).astype(np.int64).sum()) * wl.cfg.Hkv * wl.cfg.D * 2 * 2
    cores = len(os.sched_getaffinity(0))
    times, passes, work = [], 0, 0.0
    with threadpool_limits(limits=cores):
        blas_threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()
                            if p.get("user_api") == "blas"] or [1])
        ref, _ = oracle.attend(q, k, v, bt, sl, wl.cfg.scale)     # warm-up (page faults, BLAS)
        for _ in range(3):
            n, t0 = 0, time.perf_counter()
            while True:
                ref, _ = oracle.attend(q, k, v, bt, sl, wl.cfg.scale)
                n += 1
                el = time.perf_counter() - t0
                if el >= budget_s / 3 or el * (n + 1) / n > budget_s:
                    break
            times.append(el / n)
            passes += n
            work += el
    t = float(np.median(times))
    got = out_gpu.float().cpu().numpy()[rows]
    err = float(np.max(np.abs(got - ref)))
    rel = err / float(np.max(np.abs(ref)))
    return {
        "value": round(len(rows) / t, 3),
        "unit": "tokens/s",
        "kv_gbps": round(kv_bytes / t / 1e9, 3),
        "cores": blas_threads,
        "host_cores": cores,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": (f"{len(rows)} of {len(wl.seq_lens_np)} rows, all {wl.cfg.Hq} heads, "
                   f"{int(np.asarray(sl).sum())} tokens ({kv_bytes / 1e6:.1f} MB of fp16 K/V); "
                   f"float64 numpy, BLAS allowed {cores} threads (uses {blas_threads}); "
                   f"median of 3 runs, {passes} whole passes in {work:.1f} s; pages copied to "
                   f"host before timing"),
        "seconds_per_pass_runs": [round(x, 4) for x in times],
        "gpu_vs_oracle_max_abs_err": err,
        "gpu_vs_oracle_rel_err": rel,
    }


def measure(name, args, seed, kv_dtype, steps, warmup):
    """Time `steps` back-to-back steps of workload `name` through the runner
    (policy + plan + kernels), with HIP-event windows over the step's own
    kernels inside the timed region; then lone synchronised steps,
    host-planned and device-planned from a captured graph."""
    import torch

    import paged_gqa_decode_pkv_amd as pkv
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[name]
    dev = torch.device("cuda")
    print(f"[bench] drawing {cfg.name} seed {seed}", file=sys.stderr, flush=True)
    wl = make_workload(cfg, seed, device="cuda", dtype="fp8" if kv_dtype == "fp8" else "f16")
    B = len(wl.seq_lens_np)
    kv_bytes = wl.kv_bytes
    L = args.layers or max(1, min(16, math.ceil((2 << 30) / max(kv_bytes, 1))))
    if cfg.name == "b64":
        L = 1
    layers = [(wl.q, wl.k_pool, wl.v_pool)]
    for _ in range(L - 1):
        layers.append((wl.q.clone(), wl.k_pool.clone(), wl.v_pool.clone()))
    outs = [torch.empty_like(wl.q) for _ in range(L)]
    lses = [torch.empty((B, cfg.Hq), dtype=torch.float32, device=dev) for _ in range(L)]
    sl_h = wl.seq_lens_np
    # block table checked once on the host, as a serving loop does on admission
    pkv.pkv_plan(sl_h, cfg.Hkv, cfg.max_pages_per_row, 0, 1, block_table=wl.block_table_np,
                 num_pages=wl.k_pool.shape[0])
    decs = []
    for li, (q, k, v) in enumerate(layers):
        d = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=B,
                             max_pages_per_row=cfg.max_pages_per_row)
        d.set_inputs(q, k, v, wl.block_table, wl.seq_lens, sl_h, cfg.scale, outs[li], lses[li])
        decs.append(d)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        decs[i % L].run(args.mode, args.param, stream=stream, events=ev)

    print(f"[bench] {cfg.name}: warmup {warmup} steps, {L} layer copies", file=sys.stderr,
          flush=True)
    for i in range(max(warmup, L)):
        step(i)
    torch.cuda.synchronize()
    if any(d.error_flags() != 0 for d in decs):
        raise RuntimeError("device error flags set")

    K = steps
    # Event windows: window w spans `win` back-to-back steps, from the first
    # decode kernel's start to the last step's last kernel's end (the merge
    # kernel in the two-launch form); at least three windows.
    win = max(1, min(args.event_window, K // 3))
    every = max(win, min(args.event_every, K // 3))
    starts = list(range(0, K - win + 1, every))
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in starts]
    for e0, e1 in events:     # creates the underlying HIP events
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    plan_ev = {}
    for w, i0 in enumerate(starts):
        e0, e1 = events[w]
        if win == 1:
            plan_ev[i0] = (e0, e1)
        else:
            plan_ev[i0] = (e0, None)
            plan_ev[i0 + win - 1] = (None, e1)
    t0 = time.perf_counter()
    for i in range(K):
        step(i, plan_ev.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print(f"[bench] {cfg.name}: timed {K} steps", file=sys.stderr, flush=True)
    dec = decs[0]
    mode, param, T, nslots, _, two = dec.last

    # Outside the timed region: one step at a time, each waited for, as the
    # pages time a step (host policy and plan, launches, synchronisation).
    synced = []
    for i in range(min(K, 50)):
        s0 = time.perf_counter()
        step(i)
        torch.cuda.synchronize()
        synced.append((time.perf_counter() - s0) * 1e6)

    # The device-planned step (policy and plan in the decode kernel's
    # prologue), captured once per layer copy in a graph: lone synchronised
    # replays, and back-to-back replays.
    dp = None
    if not args.no_device_plan:
        need = pkv.pkv_workspace_size_device_plan(B, cfg.Hq, cfg.Hkv, cfg.D,
                                                  DEVICE_PLAN_MAX_SPLITS)
        graphs, wss = [], []
        for li, (q, k, v) in enumerate(layers):
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            pkv.pkv_workspace_init(ws)
            wss.append(ws)

            def dstep(q=q, k=k, v=v, ws=ws, li=li):
                pkv.pkv_decode_device_plan(q, k, v, wl.block_table, wl.seq_lens, cfg.scale,
                                           outs[li], ws, DEVICE_PLAN_MAX_SPLITS, lse=lses[li])
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                dstep()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                dstep()
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(2 * L):
            graphs[i % L].replay()
        torch.cuda.synchronize()
        d_synced = []
        for i in range(min(K, 50)):
            s0 = time.perf_counter()
            graphs[i % L].replay()
            torch.cuda.synchronize()
            d_synced.append((time.perf_counter() - s0) * 1e6)
        # Back to back: all layer copies in one graph, as a model's decode
        # step captures its layers (one graph launch per L steps).
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for li in range(L):
                pkv.pkv_decode_device_plan(layers[li][0], layers[li][1], layers[li][2],
                                           wl.block_table, wl.seq_lens, cfg.scale, outs[li],
                                           wss[li], DEVICE_PLAN_MAX_SPLITS, lse=lses[li])
        g_all.replay()
        torch.cuda.synchronize()
        reps = max(1, K // L)
        r0 = time.perf_counter()
        for _ in range(reps):
            g_all.replay()
        torch.cuda.synchronize()
        d_wall = (time.perf_counter() - r0) * K / (reps * L)
        hdr, _, _ = pkv.pkv_device_plan_read(wss[0], B, cfg.Hq, cfg.Hkv, cfg.D,
                                             DEVICE_PLAN_MAX_SPLITS)
        dp = {
            "synced_step_us": {"median": round(float(np.median(d_synced)), 2),
                               "p10": round(float(np.percentile(d_synced, 10)), 2),
                               "p90": round(float(np.percentile(d_synced, 90)), 2),
                               "tokens_per_s": round(B / (float(np.median(d_synced)) * 1e-6),
                                                     2)},
            "back_to_back_us_per_step": round(d_wall / K * 1e6, 2),
            "tokens_per_s": round(B * K / d_wall, 2),
            "plan": {"mode": ["split", "workqueue"][hdr["mode"]], "param": hdr["param"],
                     "tasks": hdr["num_tasks"], "fused": bool(hdr["fused"])},
            "note": "pkv_decode_device_plan (policy and plan on the GPU from device-resident "
                    f"lengths, capacity {DEVICE_PLAN_MAX_SPLITS} splits per row); synced: one "
                    "step per graph, replayed alone and waited for; back to back: the "
                    f"{L} layer copies' steps in one graph, replayed {max(1, K // L)} times",
        }

    # Explicit split counts of a single-row batch (the pages' sequence
    # splitting at S = 8..64), each in the launch form the rule gives it:
    # HIP-event time per step over three windows of 8 back-to-back steps.
    sweep = None
    if B == 1 and args.mode is None:
        sweep = {}
        for S in SPLIT_SWEEP:
            for i in range(2 * L):
                decs[i % L].run(pkv.PKV_MODE_SPLIT, S, stream=stream)
            torch.cuda.synchronize()
            per = []
            for _ in range(3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()        # creates the underlying HIP events
                e1.record()
                torch.cuda.synchronize()
                for i in range(8):
                    ev = (e0 if i == 0 else None, e1 if i == 7 else None)
                    decs[i % L].run(pkv.PKV_MODE_SPLIT, S, stream=stream, events=ev)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3 / 8)
            two_s = bool(decs[0].last[5])
            us = float(np.median(per))
            sweep[f"S={S}"] = {"step_us": round(us, 2),
                               "kv_gbps": round(kv_bytes / (us * 1e-6) / 1e9, 1),
                               "merge": "two-launch" if two_s else "fused"}
        for i in range(2 * L):     # back to the policy's plan
            step(i)
        torch.cuda.synchronize()

    wall = t1 - t0
    win_ms = np.array([e0.elapsed_time(e1) / win for e0, e1 in events])
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    fp8 = kv_dtype == "fp8"
    load_mode = pkv.pkv_page_load_mode(cfg.D, pkv.PKV_DTYPE_F16_KV_FP8 if fp8
                                       else pkv.PKV_DTYPE_F16, T, num_cus)
    two_launch = bool(two)
    avg_s = float(win_ms.mean()) * 1e-3
    achieved = kv_bytes / avg_s / 1e9
    ms_per_step = wall / K * 1e3
    splits = np.diff(dec.plan_arrays()[1])
    kernel = (f"pkv_decode_kernel<{cfg.D}, {'true' if B <= 1024 else 'false'}, _Float16, "
              f"{'pkv::Fp8E4M3' if fp8 else '_Float16'}, false, {load_mode}>")
    if two_launch:
        kernel += f" + pkv_merge_kernel<{cfg.D}, _Float16>"
    sched = {"workload": cfg.name, "seed": seed, "kv_dtype": kv_dtype,
             "mode": ["split", "workqueue"][mode], "param": param,
             "merge": "two-launch" if two_launch else "fused"}
    return wl, outs[0], {
        "B": B, "kv_bytes": kv_bytes, "K": K, "wall": wall, "ms_per_step": ms_per_step,
        "config": {
            "workload": cfg.name, "seed": seed, "B": B, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
            "head_dim": cfg.D, "page_size": 16, "kv_dtype": kv_dtype,
            "seq_lens": sl_h.tolist(), "kv_bytes_per_step": kv_bytes,
            "mode": ["split", "workqueue"][mode], "param": param, "tasks": T,
            "layers_rotated": L, "launches_per_step": 2 if two_launch else 1,
            "merge": "separate merge kernel" if two_launch else "fused into the decode kernel",
            "step": "policy + plan (host C++; a changed plan is read from pinned memory, a "
                    "repeated one from its copy in the workspace) + decode kernel (+ merge "
                    "kernel in the two-launch form)",
        },
        "kv_gbps_step": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "synced_step_us": {
            "median": round(float(np.median(synced)), 2),
            "p10": round(float(np.percentile(synced, 10)), 2),
            "p90": round(float(np.percentile(synced, 90)), 2),
            "tokens_per_s": round(B / (float(np.median(synced)) * 1e-6), 2),
            "note": "one step at a time, each followed by a synchronisation (outside the timed "
                    "region): the latency of a lone step, host policy and plan included",
        },
        "gpu_us": {
            "step_mean": round(float(win_ms.mean()) * 1e3, 2),
            "step_p10": round(float(np.percentile(win_ms, 10)) * 1e3, 2),
            "step_p90": round(float(np.percentile(win_ms, 90)) * 1e3, 2),
            "timing": f"HIP events on the step's own kernels: {len(events)} windows of {win} "
                      f"back-to-back steps, one every {every} steps, from the first decode "
                      f"kernel's start to the last step's last kernel's end; per step = "
                      f"window / {win}",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": _traffic(cfg.name, sched),
            "kernel": kernel,
            "event_windows": len(events),
            "steps_per_event_window": win,
            "algorithmic_bytes_per_launch": kv_bytes,
            "extras_bytes_per_launch": {
                "q_out_bytes": B * cfg.Hq * cfg.D * 4,
                "block_table_bytes": int(((sl_h.astype(np.int64) + 15) // 16).sum()) * 4,
                "partial_state_bytes_written": int(splits[splits > 1].sum()) * cfg.Hq
                * (cfg.D + 2) * 4,
            },
        },
        "device_planned": dp,
        "split_sweep": sweep,
        "merge_state_bytes": merge_state_bytes(cfg, sl_h, num_cus),
    }


def merge_state_bytes(cfg, lens, num_cus):
    """Merge-state traffic of the policy's best split-mode and best workqueue
    plan for this batch (each by the policy's model, whatever the mode rule
    picks): partial states written by the split tasks of rows with more than
    one split and read back by the merge, Hq x (d + 2) fp32 per slot each
    way."""
    import paged_gqa_decode_pkv_amd as pkv
    out = {}
    for mode, name, cands in ((pkv.PKV_MODE_SPLIT, "split", [2 ** k for k in range(9)]),
                              (pkv.PKV_MODE_WORKQUEUE, "workqueue",
                               [4 * 2 ** k for k in range(7)])):
        best = min(cands, key=lambda v: pkv.pkv_policy_predict(lens, cfg.Hkv, num_cus, mode, v,
                                                               head_dim=cfg.D))
        _, offs, _ = pkv.pkv_plan(lens, cfg.Hkv, cfg.max_pages_per_row, mode, best)
        sp = np.diff(offs)
        slots = int(sp[sp > 1].sum())
        out[name] = {"param": best, "partial_slots": slots,
                     "bytes": 2 * slots * cfg.Hq * (cfg.D + 2) * 4}
    sb, wb = out["split"]["bytes"], out["workqueue"]["bytes"]
    out["workqueue_vs_split"] = round(wb / sb, 4) if sb else None
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="b8_bimodal")
    ap.add_argument("--extra-workload", default="b1",
                    help="a second workload measured in the same run (key of its own); "
                         "'none' to skip")
    ap.add_argument("--kv-dtype", default="f16", choices=("f16", "fp8"),
                    help="K/V pool element type: fp16, or fp8 E4M3 codes (q and out stay fp16)")
    ap.add_argument("--seed", type=int, default=20260623)
    ap.add_argument("--mode", type=int, default=None, help="0 split / 1 workqueue (default: policy)")
    ap.add_argument("--param", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None,
                    help="KV copies rotated over (default: enough for >= 2 GiB between reuses)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (three runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-device-plan", action="store_true",
                    help="skip the graph-replayed device-planned step")
    ap.add_argument("--event-every", type=int, default=16,
                    help="start an event window on every n-th timed step (at least three "
                         "windows)")
    ap.add_argument("--event-window", type=int, default=8,
                    help="back-to-back steps per event pair: the start event takes the first "
                         "decode kernel's start, the end event the last step's last kernel's "
                         "end (a lone timed launch reads about 3 us long)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (scales PMC byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 5}), flush=True)
        return

    wl, out0, m = measure(args.workload, args, args.seed, args.kv_dtype, args.steps, args.warmup)
    res = {
        "metric": METRIC,
        "value": round(m["B"] * m["K"] / m["wall"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": m["config"],
        "kv_gbps_step": m["kv_gbps_step"],
        "synced_step_us": m["synced_step_us"],
        "gpu_us": m["gpu_us"],
        "roofline": m["roofline"],
        "device_planned": m["device_planned"],
        "split_sweep": m["split_sweep"],
        "merge_state_bytes": m["merge_state_bytes"],
    }
    # The second workload is timed right after the first, before the seconds
    # of host-only work of the CPU baseline: timed after them, the B1 step
    # read about 1 us slower (30.1 against 29.1 us per step on one box), which
    # its 40 warm-up steps did not recover.
    if args.extra_workload != "none" and args.extra_workload != args.workload:
        _, _, x = measure(args.extra_workload, args, args.seed, args.kv_dtype, args.steps,
                          args.warmup)
        res[args.extra_workload] = {
            "tokens_per_s": round(x["B"] * x["K"] / x["wall"], 2),
            "ms_per_step": round(x["ms_per_step"], 5),
            "kv_gbps_step": x["kv_gbps_step"],
            "config": x["config"],
            "synced_step_us": x["synced_step_us"],
            "gpu_us": x["gpu_us"],
            "roofline": x["roofline"],
            "device_planned": x["device_planned"],
            "split_sweep": x["split_sweep"],
            "merge_state_bytes": x["merge_state_bytes"],
        }
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        B = m["B"]
        rows = None if B <= 8 else [0, 1, 2, 3]
        res["cpu_baseline"] = cpu_baseline(wl, out0, args.cpu_budget, rows)
    else:
        res["cpu_baseline"] = None
    del wl, out0
    torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
