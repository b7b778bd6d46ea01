"""Per-workgroup timeline of the decode step (a profiling tool; GPU required).

Loads the timeline build of the library (``python -m
paged_gqa_decode_pkv_amd.build --timeline`` writes libpkv_timeline.so:
the same kernels, with realtime-counter marks kept in registers and stored
once per workgroup at its exit) and, for each workload, runs the step the
bench runs -- the host-planned step through the native runner, and the
device-planned step -- over rotated layer copies, then reads back the marks
of the last launch of a window of back-to-back steps.

Marks (per workgroup, microseconds from the launch's earliest entry):
  plan       device plan done (self-planned step only)
  issued     first page loads issued
  prologue   prologue barrier passed (q in LDS)
  first      first round of the first task consumed
  last       last round of the workgroup's last task consumed
  loop_end   task loop left
  merged     final arrivals and merges done
  exit       workgroup exit
  waves_last the last of the four waves' last rounds of the latest task
             ("last" is wave 0's)
  states_lds the waves' states in LDS, barrier passed (latest task)
  combined   the combined state of the latest task written (output or
             partial)
The summary gives each mark's median and maximum over the workgroups, the
last-round and exit times per XCD, the tasks per workgroup, and a split of
the launch into start (entry to the median first round), streaming (to the
median last round), imbalance (to the latest last round) and tail (to the
latest exit).

    python -m paged_gqa_decode_pkv_amd.timeline [--workloads b8_bimodal b1]
        [--reps 3] [--out-dir profiles]
"""
from __future__ import annotations

import argparse
import ctypes
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TIMELINE_LIB = os.path.join(HERE, "libpkv_timeline.so")
SLOTS = 16
WORKGROUPS = 4096
MARKS = ("entry", "plan", "issued", "prologue", "first", "last", "loop_end", "merged", "exit",
         "waves_last", "states_lds", "combined")
# slots of the marks in a workgroup's row (9 holds the XCD, 10 the tasks run)
MARK_SLOTS = (0, 1, 2, 3, 4, 5, 6, 7, 8, 11, 12, 13)
DEVICE_PLAN_MAX_SPLITS = 64


def _load():
    if not os.path.exists(TIMELINE_LIB):
        raise SystemExit("no timeline build: run python -m paged_gqa_decode_pkv_amd.build "
                         "--timeline first")
    sys.path.insert(0, ROOT)
    import torch  # noqa: F401  (the HIP runtime torch brings is the one the library binds to)
    import paged_gqa_decode_pkv_amd as pkv
    if pkv._lib is not None and os.path.realpath(pkv.LIB_PATH) != os.path.realpath(TIMELINE_LIB):
        raise SystemExit("the product library is already loaded in this process")
    pkv.LIB_PATH = TIMELINE_LIB     # the binding loads its library on first use
    lib = pkv._load()
    lib.pkv_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.pkv_timeline_read.restype = ctypes.c_int
    return pkv, lib


def _read(lib, grid):
    buf = np.zeros(WORKGROUPS * SLOTS, np.uint64)
    if lib.pkv_timeline_read(buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError("pkv_timeline_read failed")
    d = buf.reshape(WORKGROUPS, SLOTS)[:grid].astype(np.int64)
    t0 = d[:, 0].min()
    raw = d[:, list(MARK_SLOTS)]
    rel = (raw - t0) / 100.0               # 100 MHz counter -> us
    rel[raw == 0] = np.nan                 # marks a workgroup never reached
    return rel, d[:, 9], d[:, 10]


def _summary(rel, xcc, tasks):
    med = {m: float(np.nanmedian(rel[:, i])) if np.isfinite(rel[:, i]).any() else None
           for i, m in enumerate(MARKS)}
    mx = {m: float(np.nanmax(rel[:, i])) if np.isfinite(rel[:, i]).any() else None
          for i, m in enumerate(MARKS)}
    per_xcd = {}
    for x in sorted(set(xcc.tolist())):
        sel = xcc == x
        per_xcd[int(x)] = (float(np.nanmax(rel[sel, 5])), float(np.nanmax(rel[sel, 8])))
    split = {
        "start (to the median first round)": med["first"],
        "streaming (to the median last round)": med["last"] - med["first"],
        "imbalance (to the latest last round)": mx["last"] - med["last"],
        "tail (to the latest exit)": mx["exit"] - mx["last"],
    }
    return med, mx, per_xcd, np.bincount(tasks).tolist(), split


def run_workload(pkv, lib, name, seed, reps, window):
    import torch
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed, device="cuda")
    B = len(wl.seq_lens_np)
    L = max(1, min(16, math.ceil((2 << 30) / max(wl.kv_bytes, 1))))
    layers = [(wl.q, wl.k_pool, wl.v_pool)]
    for _ in range(L - 1):
        layers.append((wl.q.clone(), wl.k_pool.clone(), wl.v_pool.clone()))
    outs = [torch.empty_like(wl.q) for _ in range(L)]
    lses = [torch.empty((B, cfg.Hq), dtype=torch.float32, device="cuda") for _ in range(L)]
    decs = []
    for li, (q, k, v) in enumerate(layers):
        d = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=B,
                             max_pages_per_row=cfg.max_pages_per_row)
        d.set_inputs(q, k, v, wl.block_table, wl.seq_lens, wl.seq_lens_np, cfg.scale, outs[li],
                     lses[li])
        decs.append(d)
    need = pkv.pkv_workspace_size_device_plan(B, cfg.Hq, cfg.Hkv, cfg.D, DEVICE_PLAN_MAX_SPLITS)
    wss = []
    for _ in range(L):
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        pkv.pkv_workspace_init(ws)
        wss.append(ws)
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count

    def host_step(i):
        decs[i % L].run(None, None)

    def device_step(i):
        li = i % L
        q, k, v = layers[li]
        pkv.pkv_decode_device_plan(q, k, v, wl.block_table, wl.seq_lens, cfg.scale, outs[li],
                                   wss[li], DEVICE_PLAN_MAX_SPLITS, lse=lses[li])

    results = {}
    for kind, step in (("host-planned", host_step), ("device-planned", device_step)):
        for i in range(2 * L):
            step(i)
        torch.cuda.synchronize()
        if kind == "host-planned":
            mode, param, T, _, _, two = decs[0].last
            plan = (f"{['split S', 'workqueue c'][mode]}={param}, {T} tasks, "
                    f"{'two launches' if two else 'fused merge'}")
            grid = min(T, num_cus * (1 if cfg.D == 256 else 2))
        else:
            hdr, _, _ = pkv.pkv_device_plan_read(wss[0], B, cfg.Hq, cfg.Hkv, cfg.D,
                                                 DEVICE_PLAN_MAX_SPLITS)
            plan = (f"{['split S', 'workqueue c'][hdr['mode']]}={hdr['param']}, "
                    f"{hdr['num_tasks']} tasks, {'fused merge' if hdr['fused'] else 'two launches'}")
            grid = num_cus
        runs = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(window):
                step(i)
            e1.record()
            torch.cuda.synchronize()
            per_step = e0.elapsed_time(e1) * 1e3 / window
            runs.append((per_step,) + _summary(*_read(lib, grid)))
        results[kind] = (plan, grid, runs)
        print(f"[timeline] {name} {kind}: {plan}; per step "
              f"{np.median([r[0] for r in runs]):.2f} us", flush=True)
    del layers, decs, wss
    torch.cuda.empty_cache()
    return wl, results


def write_markdown(path, name, seed, kv_bytes, results, command):
    lines = [f"# Per-workgroup timeline: decode step on the {name} workload", "",
             f"Workload: {name} (seed {seed}), {kv_bytes:,} B of K+V per step; 1x MI355X "
             "(gfx950).", "",
             "Command (from the repo root; the timeline build first, on any machine):", "",
             "    python -m paged_gqa_decode_pkv_amd.build --timeline",
             f"    {command}", "",
             "Marks are microseconds from the launch's earliest workgroup entry (realtime "
             "counter, 100 MHz), one launch per repetition, the last of a window of "
             "back-to-back steps; 'per step' is the window's HIP-event time over its steps "
             "(launch gaps included).", ""]
    for kind, (plan, grid, runs) in results.items():
        lines += [f"## {kind}: {plan}, {grid} workgroups", ""]
        lines += ["| rep | per step | " + " | ".join(MARKS[1:]) + " |",
                  "|---|---|" + "---|" * (len(MARKS) - 1)]
        for r, (per_step, med, mx, per_xcd, tasks, split) in enumerate(runs):
            cells = []
            for m in MARKS[1:]:
                cells.append("-" if med[m] is None else f"{med[m]:.2f} / {mx[m]:.2f}")
            lines.append(f"| {r} | {per_step:.2f} | " + " | ".join(cells) + " |")
        lines += ["", "(each mark: median / maximum over the workgroups, us)", ""]
        per_step, med, mx, per_xcd, tasks, split = runs[-1]
        lines += ["Last repetition, per XCD (latest last round / latest exit, us): " +
                  ", ".join(f"XCD {x}: {a:.2f} / {b:.2f}" for x, (a, b) in per_xcd.items()),
                  "",
                  "Tasks per workgroup (count of workgroups with 0, 1, 2, ... tasks): "
                  f"{tasks}", "",
                  "Where the launch goes (last repetition): " +
                  "; ".join(f"{k} {v:.2f} us" for k, v in split.items()), ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workloads", nargs="*", default=["b8_bimodal", "b1"])
    ap.add_argument("--seed", type=int, default=20260623)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--window", type=int, default=8)
    ap.add_argument("--out-dir", default=None,
                    help="write decode_<workload>_timeline.md here (default: print only)")
    args = ap.parse_args(argv)
    pkv, lib = _load()
    command = ("python -m paged_gqa_decode_pkv_amd.timeline --workloads " +
               " ".join(args.workloads) + f" --seed {args.seed} --reps {args.reps} "
               f"--window {args.window}" + (f" --out-dir {args.out_dir}" if args.out_dir else ""))
    for name in args.workloads:
        wl, results = run_workload(pkv, lib, name, args.seed, args.reps, args.window)
        for kind, (plan, grid, runs) in results.items():
            per_step, med, mx, per_xcd, tasks, split = runs[-1]
            print(f"  {kind}: " + "; ".join(f"{k} {v:.2f}" for k, v in split.items()),
                  flush=True)
        if args.out_dir:
            os.makedirs(args.out_dir, exist_ok=True)
            write_markdown(os.path.join(args.out_dir, f"decode_{name}_timeline.md"), name,
                           args.seed, wl.kv_bytes, results, command)
    return 0


if __name__ == "__main__":
    sys.exit(main())
