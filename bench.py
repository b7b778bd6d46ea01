#!/usr/bin/env python3
"""Decode-step throughput of the paged GQA decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b8_bimodal]

One step is the whole hot path over one batch: the host policy and planner
(C++), the upload of the task list, the persistent decode kernel and the merge
kernel.  The batch is the B=8 bimodal workload (Hq=32, Hkv=8, d=128, page
size 16, held-out seed 20260623), drawn in HBM before timing starts.  The K/V
pool is replicated over several "layers" and the steps rotate through them,
so every step streams its KV from HBM rather than from the 256 MB
Infinity Cache.  That matches a model whose layers each own a KV cache.

Prints one JSON line: decode tokens/s (B tokens per step), KV GB/s, the
roofline of the decode kernel (HIP events on the decode kernel's own
dispatches inside the timed region) and the float64 oracle timed on host
cores as a reported baseline.
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
TRAFFIC_FILE = os.path.join(HERE, "profiles", "decode_b8_bimodal_traffic.json")


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(HERE, "paged_gqa_decode_pkv_amd", "csrc", "decode.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(config):
    """Measured HBM bytes per decode launch from the committed rocprofv3 PMC
    runs, if they were taken on the current kernel source and on this same
    workload and schedule; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != _kernel_source_hash():
        return None
    if rec.get("config") != config:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, out_gpu, budget_s: float, rows=None):
    """Time the float64 oracle (single thread) on a bounded sample of the same
    batch, and check the GPU output on that sample against it."""
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import compact_rows

    if rows is None:
        rows = list(range(len(wl.seq_lens_np)))
    q, k, v, bt, sl = compact_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, rows)
    reps = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            ref, _ = oracle.attend(q, k, v, bt, sl, wl.cfg.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or (reps >= 1 and el * (reps + 1) / reps > 3 * budget_s):
                break
    got = out_gpu.float().cpu().numpy()[rows]
    err = float(np.max(np.abs(got - ref)))
    rel = err / float(np.max(np.abs(ref)))
    return {
        "value": round(len(rows) * reps / el, 3),
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{len(rows)} of {len(wl.seq_lens_np)} rows, all {wl.cfg.Hq} heads, "
                   f"{int(sl.sum())} tokens, {reps} pass(es) in {el:.1f} s; float64 numpy, "
                   f"BLAS limited to 1 thread; pages copied to host before timing"),
        "gpu_vs_oracle_max_abs_err": err,
        "gpu_vs_oracle_rel_err": rel,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="b8_bimodal")
    ap.add_argument("--kv-dtype", default="f16", choices=("f16", "fp8"),
                    help="K/V pool element type: fp16, or fp8 E4M3 codes (q and out stay fp16)")
    ap.add_argument("--seed", type=int, default=20260623)
    ap.add_argument("--mode", type=int, default=None, help="0 split / 1 workqueue (default: policy)")
    ap.add_argument("--param", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None,
                    help="KV copies rotated over (default: enough for >= 2 GiB between reuses)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=16,
                    help="start an event window on every n-th timed step")
    ap.add_argument("--event-window", type=int, default=8,
                    help="back-to-back decode launches per event pair in the fused form: the "
                         "start event takes the first dispatch's start, the end event the last "
                         "one's end (a lone timed launch reads about 3 us long); the two-launch "
                         "form times single decode launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (scales PMC byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_gqa_decode_pkv_amd as pkv
    from workloads import CONFIGS, make_workload

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
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda")
    print(f"[bench] drawing {cfg.name} seed {args.seed}", file=sys.stderr, flush=True)
    wl = make_workload(cfg, args.seed, device="cuda",
                       dtype="fp8" if args.kv_dtype == "fp8" else "f16")
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
    num_pages = wl.k_pool.shape[0]
    sl_h = wl.seq_lens_np
    bt_h = wl.block_table_np
    # block table checked once on the host, as a serving loop does on admission
    pkv.pkv_plan(sl_h, cfg.Hkv, cfg.max_pages_per_row, 0, 1, block_table=bt_h, num_pages=num_pages)
    decs = []
    for li, (q, k, v) in enumerate(layers):
        d = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=B,
                             max_pages_per_row=cfg.max_pages_per_row)
        d.set_inputs(q, k, v, wl.block_table, wl.seq_lens, sl_h, cfg.scale, outs[li], lses[li])
        decs.append(d)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        decs[i % L].run(args.mode, args.param, stream=stream, events=ev)

    every = max(1, args.event_every)

    print(f"[bench] warmup {args.warmup} steps, {L} layer copies", file=sys.stderr, flush=True)
    for i in range(max(args.warmup, L)):
        step(i)
    torch.cuda.synchronize()
    if any(d.error_flags() != 0 for d in decs):
        print("device error flags set", file=sys.stderr)
        sys.exit(1)

    K = args.steps
    # Event windows: window w starts at step w*every and spans `win` decode
    # launches (one in the two-launch form, whose merge kernels would fall
    # inside a longer window).
    win = 1 if bool(decs[0].last[5]) else max(1, min(args.event_window, every, K))
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
    print(f"[bench] timed {K} steps", file=sys.stderr, flush=True)
    dec = decs[0]

    # Outside the timed region: one step at a time, each waited for, as the
    # pages time a step (host policy and plan, launches, synchronisation).
    synced = []
    for i in range(min(K, 50)):
        s0 = time.perf_counter()
        step(i)
        torch.cuda.synchronize()
        synced.append((time.perf_counter() - s0) * 1e6)
    synced = np.array(synced)

    wall = t1 - t0
    dec_ms = np.array([e0.elapsed_time(e1) / win for e0, e1 in events])
    mode, param, T, nslots = dec.last[:4]
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    # the page loads' cache policy the library gives this plan (0: default,
    # 1: non-temporal V loads, 2: non-temporal K and V loads)
    fp8 = args.kv_dtype == "fp8"
    load_mode = pkv.pkv_page_load_mode(cfg.D, pkv.PKV_DTYPE_F16_KV_FP8 if fp8 else pkv.PKV_DTYPE_F16,
                                       T, num_cus)
    two_launch = bool(dec.last[5])
    avg_dec_s = float(dec_ms.mean()) * 1e-3
    achieved = kv_bytes / avg_dec_s / 1e9
    ms_per_step = wall / K * 1e3
    splits = np.diff(dec.plan_arrays()[1])
    extras = {
        "q_out_bytes": B * cfg.Hq * cfg.D * 4,
        "block_table_bytes": int(((sl_h.astype(np.int64) + 15) // 16).sum()) * 4,
        "partial_state_bytes_written": int(splits[splits > 1].sum()) * cfg.Hq * (cfg.D + 2) * 4,
    }
    res = {
        "metric": METRIC,
        "value": round(B * K / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "seed": args.seed, "B": B, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
            "head_dim": cfg.D, "page_size": 16, "kv_dtype": args.kv_dtype,
            "seq_lens": sl_h.tolist(),
            "kv_bytes_per_step": kv_bytes, "mode": ["split", "workqueue"][mode], "param": param,
            "tasks": T, "layers_rotated": L, "launches_per_step": 2 if two_launch else 1,
            "merge": "separate merge kernel" if two_launch else "fused into the decode kernel",
            "step": "policy + plan (host C++; a changed plan is read from pinned memory, a repeated "
                    "one from the runner's device copy) "
                    "+ decode kernel (+ merge kernel in the two-launch form)",
        },
        "kv_gbps_step": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "synced_step_us": {
            "median": round(float(np.median(synced)), 2),
            "p10": round(float(np.percentile(synced, 10)), 2),
            "p90": round(float(np.percentile(synced, 90)), 2),
            "note": "one step at a time, each followed by a synchronisation (outside the timed "
                    "region): the latency of a lone step, host policy and plan included",
        },
        "gpu_us": {
            "decode_mean": round(float(dec_ms.mean()) * 1e3, 2),
            "decode_p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
            "decode_p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
            "timing": f"HIP events on the decode dispatches: {len(events)} windows of {win} "
                      f"back-to-back launch(es), one every {every} steps; per launch = "
                      f"window / {win}",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": _traffic({"workload": cfg.name, "seed": args.seed,
                                 "kv_dtype": args.kv_dtype,
                                 "mode": ["split", "workqueue"][mode], "param": param,
                                 "merge": "two-launch" if two_launch else "fused"}),
            "kernel": f"pkv_decode_kernel<{cfg.D}, {'true' if B <= 1024 else 'false'}, _Float16, "
                      f"{'pkv::Fp8E4M3' if fp8 else '_Float16'}, false, {load_mode}>",
            "event_windows": len(events),
            "launches_per_event_window": win,
            "algorithmic_bytes_per_launch": kv_bytes,
            "extras_bytes_per_launch": extras,
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        rows = None if B <= 8 else [0, 1, 2, 3]
        res["cpu_baseline"] = cpu_baseline(wl, outs[0], args.cpu_budget, rows)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
