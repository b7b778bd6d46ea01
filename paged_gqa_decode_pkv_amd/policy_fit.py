"""Fit the policy's cost model on the calibration seed; judge it on held-out seeds.

The pages describe the policy as calibrated ("2. Calibrated Adaptive Policy"
in the gist.science explainer) and roofline-style (the v2 abstract), with its
thresholds fixed on a calibration seed and then evaluated on held-out seeds
("Resultaten").  This module is the CPU half of that protocol:

  runs     the measurements of ``calibrate.py`` (every candidate schedule of
           every trace, seed 20260622 and the five held-out seeds)
  fit      least squares on log time, calibration seed only, of the model
           documented at ``pkv_policy`` in include/pkv.h
  judge    for every (trace, seed): the schedule the fitted policy picks,
           its measured time, the best measured schedule, and the regret
           (picked / best); also the regret of the runner's own pick during the
           runs (the policy the library held when they were taken)

``python -m paged_gqa_decode_pkv_amd.policy_fit --revalidate RUNS.jsonl [--name F]``
judges the committed constants on fresh runs instead (``calibration/F``, by default
``mi355x_revalidation.json``; fp8-pool runs are judged with the model pricing a page as
a 2-byte page, as the runner does).
``python -m paged_gqa_decode_pkv_amd.policy_fit RUNS.jsonl`` writes
``calibration/mi355x_runs.json`` (the runs, compacted) and
``calibration/mi355x_fit.json`` (constants + evaluation) and prints the table.
``--runs calibration/mi355x_runs.json`` re-fits from the committed runs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
from collections import defaultdict

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CAL_DIR = os.path.join(HERE, "calibration")
CALIBRATION_SEED = 20260622
PAGE = 16

# Candidate sets and the fused/two-launch rule of the runner (the defaults of
# pkv_policy_params).
SPLIT_MAX = 256
CHUNK_MIN = 4
CHUNK_MAX = 256
FUSE_MAX_SPLITS = 16
FUSE_MAX_GROUP_SPLITS = 256
WG_PER_CU = 2          # the decode kernel's grid: min(T, 2 * CUs)

PARAM_NAMES = ("t0_us", "t_round_us", "alpha", "cu_gbps", "hbm_gbps", "t_two_us",
               "t_two_split_us", "t_fused_split_us")


def two_launch_rule(maxS, groups):
    """The launch form the policy takes: two launches when the deepest row
    has more than FUSE_MAX_SPLITS splits and groups x those splits exceed
    FUSE_MAX_GROUP_SPLITS."""
    return maxS > FUSE_MAX_SPLITS and groups * maxS > FUSE_MAX_GROUP_SPLITS


def plan_features(lens, Hkv, mode, param):
    """(T, P, pmax, maxS) of a plan, in closed form: T tasks, P page tiles in
    all, pmax the largest task in pages, maxS the most splits of one row."""
    T = P = pmax = maxS = 0
    for N in lens:
        n = -(-int(N) // PAGE)
        if n == 0:
            continue
        c = -(-n // param) if mode == 0 else param
        S = -(-n // c)
        T += Hkv * S
        P += Hkv * n
        pmax = max(pmax, min(c, n))
        maxS = max(maxS, S)
    return T, P, pmax, maxS


def predict(x, T, P, pmax, maxS, two, cus, head_dim):
    """Model time (us) of one step; the same formula, in the same order of
    operations, as pkv_policy in csrc/plan.cpp."""
    t0, t_round, alpha, cu_gbps, hbm_gbps, t_two, t_two_split, t_fused_split = x
    if T == 0:
        return t0
    W = min(T, WG_PER_CU * cus)
    A = min(W, cus)
    rho = min(cu_gbps, hbm_gbps / A)
    if T <= W:
        load = float(-(-T // A) * pmax)
    else:
        load = P / A + alpha * pmax
    tile = 2.0 * PAGE * head_dim * 2.0
    t = t0 + t_round * (-(-T // W)) + load * tile / (rho * 1e3)
    if two:
        t = t + t_two + t_two_split * maxS
    else:
        t = t + t_fused_split * maxS
    return t


def candidates(lens):
    """The candidates pkv_policy searches: split counts for a single active
    row, workqueue chunks for a batch (the explainer's mode rule)."""
    if sum(1 for n in lens if int(n) > 0) <= 1:
        S = 1
        while S <= SPLIT_MAX:
            yield 0, S
            S *= 2
    else:
        c = CHUNK_MIN
        while c <= CHUNK_MAX:
            yield 1, c
            c *= 2


def pick(x, lens, Hkv, cus, head_dim):
    best = None
    for mode, param in candidates(lens):
        T, P, pmax, maxS = plan_features(lens, Hkv, mode, param)
        groups = Hkv * sum(1 for n in lens if int(n) > 0)
        two = two_launch_rule(maxS, groups)
        t = predict(x, T, P, pmax, maxS, two, cus, head_dim)
        if best is None or t < best[0]:
            best = (t, mode, param, two)
    return best[1:]


# --------------------------------------------------------------------------- data

def compact_runs(jsonl_path):
    runs = defaultdict(dict)
    dtypes = set()
    for line in open(jsonl_path):
        r = json.loads(line)
        dtypes.add(r.get("dtype", "f16"))
        key = r["config"]
        d = runs[key].setdefault(str(r["seed"]), {"lens": r["lens"], "runs": [], "rule": None})
        row = [r["mode"], r["param"], int(r["two_launch"]), r["num_tasks"], r["max_splits"],
               r["step_us"]]
        if r["requested"] is None:
            d["rule"] = row
        else:
            d["runs"].append(row)
    assert len(dtypes) == 1, dtypes
    dtype = dtypes.pop()
    # fp8 pools are priced as 2-byte pools of the same head dimension, as the
    # runner and the device planner pass it
    head_dim = 128
    return {"device": "1x MI355X (gfx950), 256 CUs", "Hkv": 8, "head_dim": head_dim, "cus": 256,
            "dtype": dtype,
            "columns": ["mode", "param", "two_launch", "num_tasks", "max_splits", "step_us"],
            "command": "python -m paged_gqa_decode_pkv_amd.calibrate --out RUNS.jsonl",
            "traces": runs}


def records(data):
    """One record per measured candidate.  The time is the "step_us" column
    (steady-state time per step), or "gpu_us" in runs taken before it existed
    (HIP events from the decode kernel to the end of the step)."""
    cols = data["columns"]
    ti = cols.index("step_us") if "step_us" in cols else cols.index("gpu_us")
    out = []
    for cfg, seeds in data["traces"].items():
        for seed, d in seeds.items():
            for row in d["runs"]:
                mode, param, two, T, maxS = row[:5]
                step = row[ti]
                Tf, P, pmax, mS = plan_features(d["lens"], data["Hkv"], mode, param)
                assert (Tf, mS) == (T, maxS), (cfg, seed, mode, param)
                groups = data["Hkv"] * sum(1 for n in d["lens"] if int(n) > 0)
                out.append(dict(cfg=cfg, seed=int(seed), mode=mode, param=param, two=bool(two),
                                T=T, P=P, pmax=pmax, maxS=maxS, groups=groups, step=step))
    return out


def fit(recs, cus, head_dim):
    from scipy.optimize import least_squares
    # The launch form of a candidate is fixed by the rule, so the model is
    # fitted on the runs in that form: the only ones the policy can pick.
    cal = [r for r in recs if r["seed"] == CALIBRATION_SEED and
           r["two"] == two_launch_rule(r["maxS"], r["groups"])]

    def resid(x):
        return np.array([math.log(predict(x, r["T"], r["P"], r["pmax"], r["maxS"], r["two"],
                                          cus, head_dim)) - math.log(r["step"]) for r in cal])
    x0 = [10.0, 5.0, 0.5, 40.0, 6000.0, 5.0, 0.01, 0.3]
    lb = [0.0, 0.0, 0.0, 1.0, 500.0, 0.0, 0.0, 0.0]
    ub = [200.0, 100.0, 4.0, 1000.0, 20000.0, 100.0, 10.0, 20.0]
    sol = least_squares(resid, x0, bounds=(lb, ub))
    # round to 4 significant digits: these are the published defaults (a
    # constant that the fit drives onto its lower bound of 0 is published as 0)
    x = [0.0 if abs(v) < 1e-9 else float(f"{v:.4g}") for v in sol.x]
    return x, float(np.sqrt(np.mean(resid(x) ** 2)))


def judge(x, data, recs):
    cus, head_dim, Hkv = data["cus"], data["head_dim"], data["Hkv"]
    cols = data["columns"]
    ti = cols.index("step_us") if "step_us" in cols else cols.index("gpu_us")
    by = defaultdict(dict)
    for r in recs:
        by[(r["cfg"], r["seed"])][(r["mode"], r["param"], r["two"])] = r
    rows = []
    for cfg, seeds in data["traces"].items():
        for seed, d in seeds.items():
            runs = by[(cfg, int(seed))]
            mode, param, two = pick(x, d["lens"], Hkv, cus, head_dim)
            got = runs[(mode, param, two)]
            best = min(runs.values(), key=lambda r: r["step"])
            rule = d["rule"]
            rule_t = rule[ti] if rule else None
            rows.append({
                "trace": cfg, "seed": int(seed), "pick": [mode, param, int(two)],
                "pick_us": got["step"], "best": [best["mode"], best["param"], int(best["two"])],
                "best_us": best["step"], "regret": round(got["step"] / best["step"], 4),
                "rule": rule[:3] if rule else None,
                "rule_regret": round(rule_t / best["step"], 4) if rule else None,
            })
    return rows


def revalidate(jsonl, out_name="mi355x_revalidation.json"):
    """Judge the committed constants (no new fit) on fresh runs of calibrate.py,
    e.g. after a kernel change: for every (trace, seed), the committed policy's
    pick, its measured time and the regret against the best measured schedule;
    the constants a fit on the fresh calibration seed would give, and theirs."""
    data = compact_runs(jsonl)
    recs = records(data)
    committed = json.load(open(os.path.join(CAL_DIR, "mi355x_fit.json")))["params"]
    x = [committed[k] for k in PARAM_NAMES]
    rows = judge(x, data, recs)
    refit, rms = fit(recs, data["cus"], data["head_dim"])
    rows_refit = judge(refit, data, recs)
    held = [r["regret"] for r in rows if r["seed"] != CALIBRATION_SEED]
    held_refit = [r["regret"] for r in rows_refit if r["seed"] != CALIBRATION_SEED]
    summary = {
        "what": "committed constants judged on fresh runs (no refit); a refit shown beside them",
        "params": committed,
        "held_out_regret_mean": round(float(np.mean(held)), 4),
        "held_out_regret_max": round(float(np.max(held)), 4),
        "refit_params": dict(zip(PARAM_NAMES, refit)),
        "refit_held_out_regret_mean": round(float(np.mean(held_refit)), 4),
        "refit_held_out_regret_max": round(float(np.max(held_refit)), 4),
        "runs": data,
        "rows": rows,
    }
    with open(os.path.join(CAL_DIR, out_name), "w") as f:
        json.dump(summary, f, separators=(",", ":"))
    return summary


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("jsonl", nargs="?", help="output of calibrate.py")
    ap.add_argument("--runs", help="compacted runs (calibration/mi355x_runs.json)")
    ap.add_argument("--revalidate", action="store_true",
                    help="judge the committed constants on the runs in JSONL (no new fit)")
    ap.add_argument("--name", default="mi355x_revalidation.json",
                    help="output file (in calibration/) of --revalidate")
    args = ap.parse_args(argv)
    if args.revalidate:
        s = revalidate(args.jsonl, args.name)
        print({k: v for k, v in s.items() if k not in ("rows", "runs")})
        return 0
    if args.jsonl:
        data = compact_runs(args.jsonl)
        os.makedirs(CAL_DIR, exist_ok=True)
        with open(os.path.join(CAL_DIR, "mi355x_runs.json"), "w") as f:
            json.dump(data, f, separators=(",", ":"))
    else:
        data = json.load(open(args.runs or os.path.join(CAL_DIR, "mi355x_runs.json")))
    recs = records(data)
    x, rms = fit(recs, data["cus"], data["head_dim"])
    rows = judge(x, data, recs)
    held = [r["regret"] for r in rows if r["seed"] != CALIBRATION_SEED]
    held_rule = [r["rule_regret"] for r in rows if r["seed"] != CALIBRATION_SEED and r["rule_regret"]]
    summary = {
        "params": dict(zip(PARAM_NAMES, x)),
        "fit_rms_log_error_calibration_seed": round(rms, 4),
        "held_out_regret_mean": round(float(np.mean(held)), 4),
        "held_out_regret_max": round(float(np.max(held)), 4),
        "runner_pick_held_out_regret_mean": round(float(np.mean(held_rule)), 4) if held_rule else None,
        "runner_pick_held_out_regret_max": round(float(np.max(held_rule)), 4) if held_rule else None,
        "rows": rows,
    }
    with open(os.path.join(CAL_DIR, "mi355x_fit.json"), "w") as f:
        json.dump(summary, f, indent=1)
    name = lambda m: f"{'S' if m[0] == 0 else 'c'}={m[1]}{'/2L' if m[2] else ''}"
    print("params:", json.dumps(summary["params"]))
    print(f"{'trace':12s} {'seed':8s} {'pick':10s} {'us':>8s} {'best':10s} {'us':>8s} {'regret':>7s} {'runner pick':>11s}")
    for r in rows:
        print(f"{r['trace']:12s} {r['seed']} {name(r['pick']):10s} {r['pick_us']:8.1f} "
              f"{name(r['best']):10s} {r['best_us']:8.1f} {r['regret']:7.3f} "
              f"{r['rule_regret'] if r['rule_regret'] else float('nan'):11.3f}")
    print({k: v for k, v in summary.items() if k != "rows"})


if __name__ == "__main__":
    sys.exit(main())
