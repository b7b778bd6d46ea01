"""Policy calibration: measure every candidate schedule on the trace families.

The pages' protocol ("Evaluatieprotocol" and "Resultaten" in the gist.science
explainer): thresholds are fixed on a calibration seed (20260622) and the
policy is then judged on held-out seeds.  This tool runs the measurement half
on the GPU.  For each trace configuration and seed it draws the batch, then
times every candidate schedule through the native runner:

  split mode      S in 1, 2, 4, ..., 256
  workqueue mode  c in 4, 8, ..., 256 pages
  each in the fused single launch and, where some row has more than one
  split, in the two-launch form (decode kernel, then merge kernel)

plus the step the policy picks by itself.  The time kept per candidate is

  step_us  the wall time of K steps run back to back through the native runner
           (policy, plan, launches), synchronised only before and after,
           divided by K; the K/V pools are rotated over several copies so that
           no step reads from the 256 MB last-level cache what the step before
           it loaded.  A step costs the host about 6 us, far less than its GPU
           time, so this is the GPU's time per step: the bench's own measure.
           The median over 5 repetitions of the K steps is kept.

Output: one JSON object per line.  ``python -m paged_gqa_decode_pkv_amd.calibrate
--out FILE [--dtype f16|bf16|fp8|bf16_fp8]`` (GPU required; the constants are
fitted on fp16 runs, other element types serve to judge them).  The fit of the policy's constants from these
measurements is done by ``policy_fit.py`` on the CPU.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

TRACES = ("b1_bucketed", "b1", "b4_bimodal", "b8_bimodal", "b8_zipf", "b8_uniform",
          "b32_uniform", "b64")
SPLITS = (1, 2, 4, 8, 16, 32, 64, 128, 256)
CHUNKS = (4, 8, 16, 32, 64, 128, 256)


def measure_config(name: str, seed: int, steps: int, out_f, dtype: str = "f16"):
    import torch

    import paged_gqa_decode_pkv_amd as pkv
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed, device="cuda", fill="zero", dtype=dtype)
    B = cfg.B
    L = max(1, min(16, -(-2 * 2 ** 30 // max(wl.kv_bytes, 1))))
    pools = [(wl.k_pool, wl.v_pool)] + [(wl.k_pool.clone(), wl.v_pool.clone())
                                        for _ in range(L - 1)]
    decs = []
    for k, v in pools:
        d = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=B,
                             max_pages_per_row=cfg.max_pages_per_row)
        out = torch.empty_like(wl.q)
        lse = torch.empty(B, cfg.Hq, device="cuda")
        d.set_inputs(wl.q, k, v, wl.block_table, wl.seq_lens, wl.seq_lens_np, cfg.scale, out,
                     lse)
        decs.append(d)
    lens = wl.seq_lens_np.tolist()

    cands = [(None, None, None)]
    for S in SPLITS:
        cands += [(pkv.PKV_MODE_SPLIT, S, False), (pkv.PKV_MODE_SPLIT, S, True)]
    for c in CHUNKS:
        cands += [(pkv.PKV_MODE_WORKQUEUE, c, False), (pkv.PKV_MODE_WORKQUEUE, c, True)]

    stream = torch.cuda.current_stream()
    n = max(steps, 2 * L)
    for mode, param, two in cands:
        # plan facts
        m, p, T, slots, _, _ = decs[0].run(mode, param, two_launch=two)
        torch.cuda.synchronize()
        offs = decs[0].plan_arrays()[1]
        max_splits = int(np.max(np.diff(offs))) if B else 0
        if two and max_splits <= 1 and mode is not None:
            continue      # the merge kernel would have nothing to do
        for i in range(2 * L):
            decs[i % L].run(mode, param, stream=stream, two_launch=two)
        torch.cuda.synchronize()
        reps = []
        for _ in range(5):
            t0 = time.perf_counter()
            for i in range(n):
                decs[i % L].run(mode, param, stream=stream, two_launch=two)
            torch.cuda.synchronize()
            reps.append((time.perf_counter() - t0) / n * 1e6)
        errs = [d.error_flags() for d in decs[:1]]
        rec = {
            "config": name, "seed": seed, "B": B, "lens": lens,
            "requested": None if mode is None else [int(mode), int(param), bool(two)],
            "mode": int(m), "param": int(p), "two_launch": bool(decs[0].last[5]),
            "num_tasks": int(T), "num_partial_slots": int(slots), "max_splits": max_splits,
            "step_us": round(float(np.median(reps)), 3),
            "step_us_min": round(float(np.min(reps)), 3),
            "step_us_max": round(float(np.max(reps)), 3),
            "layers": L, "steps": n, "error_flags": errs,
            "kv_bytes": int(wl.kv_bytes),
            "dtype": dtype,
        }
        out_f.write(json.dumps(rec) + "\n")
        out_f.flush()
    del decs, pools, wl
    torch.cuda.empty_cache()


def main(argv=None):
    from workloads import CALIBRATION_SEED, HELD_OUT_SEEDS

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", required=True)
    ap.add_argument("--configs", nargs="*", default=list(TRACES))
    ap.add_argument("--seeds", nargs="*", type=int,
                    default=[CALIBRATION_SEED] + list(HELD_OUT_SEEDS))
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--dtype", default="f16", choices=("f16", "bf16", "fp8", "bf16_fp8"),
                    help="element types of q/out and the pools (workloads.make_workload)")
    args = ap.parse_args(argv)
    with open(args.out, "a") as f:
        for name in args.configs:
            for seed in args.seeds:
                t0 = time.perf_counter()
                measure_config(name, seed, args.steps, f, args.dtype)
                print(f"[calibrate] {name} seed {seed}: {time.perf_counter() - t0:.1f} s",
                      flush=True)


if __name__ == "__main__":
    sys.exit(main())
