"""Second implementation of the library's scheduling cost model -- a
cross-implementation check, NOT part of the oracle.

The schedule (split count S or workqueue chunk c, fused or two-launch merge)
changes how the decode step is computed, never its result, so the float64
oracle (``oracle/``) holds no scheduling policy.  This module re-implements,
from the formula documented at ``pkv_policy`` in include/pkv.h, the policy the
library runs, so that tests can check the C++ (and, through it, the device
planner) against an independent transcription: the same candidates in the
same order, the same float64 operations.

What pins the policy to the pages is separate (``tests/test_policy.py``): the
gist.science explainer ("Technische Samenvatting" > "2. Calibrated Adaptive
Policy") routes one long row to sequence splitting and a batch of long ragged
rows to the compact workqueue, and the tests assert exactly that decision.
The constants below are the library's own least-squares fit to MI355X step
times on the calibration seed (``paged_gqa_decode_pkv_amd/calibration/``):
parity unpinned -- nothing on the pages fixes them; their evidence is the
held-out regret recorded with the fit.
"""
from __future__ import annotations

MODE_SPLIT = 0
MODE_WORKQUEUE = 1

# The library's pkv_policy_defaults (a test keeps the three copies equal:
# this one, the C++ defaults and the committed fit).
POLICY_DEFAULTS = dict(split_max=256, chunk_min=4, chunk_max=256, fuse_max_splits=16,
                       fuse_max_group_splits=256,
                       t0_us=2.309, t_round_us=4.153, alpha=1.145, cu_gbps=46.34,
                       hbm_gbps=8667.0, t_two_us=6.018, t_two_split_us=0.0436,
                       t_fused_split_us=0.2422)


def plan_shape(seq_lens, Hkv, page_size, mode, param):
    """(T, P, pmax, maxS, groups) of the plan: tasks, page tiles in all,
    pages of the largest task, splits of the deepest row, (row, KV head)
    groups with work (closed form of the task list)."""
    T = P = pmax = maxS = groups = 0
    for N in seq_lens:
        n = -(-int(N) // page_size)
        if n == 0:
            continue
        c = -(-n // param) if mode == MODE_SPLIT else int(param)
        S = -(-n // c)
        T += Hkv * S
        P += Hkv * n
        groups += Hkv
        pmax = max(pmax, min(c, n))
        maxS = max(maxS, S)
    return T, P, pmax, maxS, groups


def two_launch(shape, k):
    """The launch form rule: two launches when the deepest row has more than
    fuse_max_splits splits and groups x those splits exceed
    fuse_max_group_splits."""
    maxS, groups = shape[3], shape[4]
    return maxS > k["fuse_max_splits"] and groups * maxS > k["fuse_max_group_splits"]


def predict_us(shape, num_cus, head_dim, page_size, two, k):
    """Model time (us) of one step of a plan shape, operation by operation as
    include/pkv.h documents it: W = min(T, 2 num_cus) workgroups, A = min(W,
    num_cus) CUs, per-CU rate min(cu_gbps, hbm_gbps / A), the critical CU's
    load, a fixed time per round of tasks, and the merge term of the launch
    form."""
    T, P, pmax, maxS = shape[:4]
    if T == 0:
        return k["t0_us"]
    W = min(T, 2 * num_cus)
    A = min(W, num_cus)
    rho = min(k["cu_gbps"], k["hbm_gbps"] / A)
    if T <= W:
        load = float(-(-T // A) * pmax)
    else:
        load = P / A + k["alpha"] * pmax
    tile = 2.0 * page_size * head_dim * 2.0
    t = k["t0_us"] + k["t_round_us"] * (-(-T // W)) + load * tile / (rho * 1e3)
    if two:
        t = t + k["t_two_us"] + k["t_two_split_us"] * maxS
    else:
        t = t + k["t_fused_split_us"] * maxS
    return t


def policy(seq_lens, Hkv, page_size, num_cus, head_dim=128, **overrides):
    """(mode, param) the library's policy picks: the mode by the explainer's
    rule (one active row: split; several: workqueue), the parameter by the
    model, first fastest candidate in ascending order.  No active row gives
    (split, 1)."""
    k = dict(POLICY_DEFAULTS)
    k.update(overrides)
    active = sum(1 for x in seq_lens if int(x) > 0)
    if active == 0:
        return MODE_SPLIT, 1
    cands = []
    if active == 1:
        S = 1
        while S <= k["split_max"]:
            cands.append((MODE_SPLIT, S))
            S *= 2
    else:
        c = k["chunk_min"]
        while c <= k["chunk_max"]:
            cands.append((MODE_WORKQUEUE, c))
            c *= 2
    best = None
    for mode, param in cands:
        shape = plan_shape(seq_lens, Hkv, page_size, mode, param)
        t = predict_us(shape, num_cus, head_dim, page_size, two_launch(shape, k), k)
        if best is None or t < best[0]:
            best = (t, mode, param)
    return best[1], best[2]
