"""The scheduling policy (host C++ ``pkv_policy``; the device planner takes
the same decision, checked on the GPU).

Source: gist.science explainer, "Technische Samenvatting" > "2. Calibrated
Adaptive Policy": one long row is decoded with sequence splitting, a batch of
eight or more long ragged rows with the compact workqueue, with thresholds
calibrated on one seed.  The pages' rule fixes the *mode*; the split count or
chunk comes from this library's cost model, whose constants are its own fit
to MI355X timings (parity unpinned -- the held-out regret recorded in
calibration/ is their evidence).  The schedule never changes the result, so
the oracle holds no policy; ``policy_model_check`` is a second transcription
of the documented model, used as a cross-implementation check only.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from tests import policy_model_check as pmc
import paged_gqa_decode_pkv_amd as pkv
from workloads import CONFIGS, CALIBRATION_SEED, HELD_OUT_SEEDS, make_lengths

SEEDS = (CALIBRATION_SEED,) + HELD_OUT_SEEDS
CUS = 256


@pytest.mark.parametrize("name", ["b1", "b1_bucketed"])
def test_one_long_row_is_split_across_the_chip(name):
    """One long row -> sequence splitting, with at least one task per CU (the
    split is what fills the chip at B = 1)."""
    for seed in SEEDS:
        lens = make_lengths(CONFIGS[name], seed)
        mode, param = pkv.pkv_policy(lens, 8, CUS)
        assert mode == pkv.PKV_MODE_SPLIT, (name, seed, mode, param)
        tasks, offs, _ = pkv.pkv_plan(lens, 8, CONFIGS[name].max_pages_per_row, mode, param)
        assert len(tasks) >= CUS // 2, (name, seed, param, len(tasks))
        if name == "b1":   # 32K tokens: enough pages to give every CU a task
            assert len(tasks) >= CUS, (seed, param, len(tasks))


@pytest.mark.parametrize("name", ["b8_bimodal", "b8_zipf", "b8_uniform", "b4_bimodal",
                                  "b32_uniform", "b64"])
def test_batches_of_long_ragged_rows_use_the_workqueue(name):
    """B >= 8 long ragged rows -> the compact workqueue, on the calibration
    seed and all five held-out seeds (B = 4, which the pages hand to another
    library, takes the workqueue here)."""
    for seed in SEEDS:
        lens = make_lengths(CONFIGS[name], seed)
        mode, param = pkv.pkv_policy(lens, 8, CUS)
        assert mode == pkv.PKV_MODE_WORKQUEUE, (name, seed, mode, param)
        assert 4 <= param <= 256 and param & (param - 1) == 0


def test_policy_mode_rule_edges():
    assert pkv.pkv_policy([0, 0], 8, CUS) == (pkv.PKV_MODE_SPLIT, 1)      # nothing to do
    assert pkv.pkv_policy([], 8, CUS) == (pkv.PKV_MODE_SPLIT, 1)
    m, p = pkv.pkv_policy([0, 40000, 0], 8, CUS)                           # one active row
    assert m == pkv.PKV_MODE_SPLIT and p >= 2
    m, p = pkv.pkv_policy([100, 0], 8, CUS)
    assert m == pkv.PKV_MODE_SPLIT
    m, p = pkv.pkv_policy([16, 16], 8, CUS)                                # two rows
    assert m == pkv.PKV_MODE_WORKQUEUE
    # a short row: never more tasks than (page, KV head) tiles
    m, p = pkv.pkv_policy([100, 0], 8, CUS)
    tasks, _, _ = pkv.pkv_plan([100, 0], 8, 8, m, p)
    assert 8 <= len(tasks) <= 8 * 7


@pytest.mark.parametrize("seed", range(6))
def test_plan_shape_pinned_to_the_task_list(seed):
    """The model's plan-shape closed form equals what the oracle's enumerated
    task list (and a page-walking enumerator) holds."""
    rng = np.random.default_rng(400 + seed)
    lens = rng.integers(0, 5000, size=int(rng.integers(1, 12)))
    lens[rng.integers(0, len(lens))] = 0
    for mode, params in ((oracle.MODE_SPLIT, (1, 2, 5, 64)),
                         (oracle.MODE_WORKQUEUE, (1, 3, 16, 999))):
        for p in params:
            tasks, offs = oracle.plan_tasks(lens, 3, 16, mode, p)
            walk = brute.tasks_by_walking(lens, 3, 16, (lambda b, n: -(-n // p)) if mode == 0
                                          else (lambda b, n: p))
            assert [tuple(t) for t in tasks] == [tuple(t) for t in walk]
            n = [-(-int(x) // 16) for x in lens]
            pages = [min((s + 1) * c, n[b]) - s * c for b, g, s, c in walk]
            T, P, pmax, maxS, groups = pmc.plan_shape(lens, 3, 16, mode, p)
            assert (T, P, pmax) == (len(walk), sum(pages), max(pages, default=0))
            assert groups == len({(b, g) for b, g, s, c in walk})
            assert maxS == max((offs[i + 1] - offs[i] for i in range(len(lens))), default=0)


def test_predict_us_closed_forms():
    """Special cases of the documented time model that reduce to plain
    arithmetic, checked on the library's own pkv_policy_predict."""
    k = pmc.POLICY_DEFAULTS
    d = pkv.pkv_policy_defaults()
    # one row of 10 pages, split S = 1 at Hkv = 1: one task on one CU at the smaller rate
    t = pkv.pkv_policy_predict([160], 1, CUS, pkv.PKV_MODE_SPLIT, 1, 0)
    rho = min(d.cu_gbps, d.hbm_gbps / 1)
    want = d.t0_us + d.t_round_us + 10 * 8192 / (rho * 1e3) + d.t_fused_split_us
    assert abs(t - want) < 1e-9
    # 512 equal tasks of 20 pages fill 2 x 256 workgroups: load = 2 tasks per CU
    t = pkv.pkv_policy_predict([320] * 64, 8, CUS, pkv.PKV_MODE_WORKQUEUE, 20, 0)
    rho = min(d.cu_gbps, d.hbm_gbps / 256)
    want = d.t0_us + d.t_round_us + 40 * 8192 / (rho * 1e3) + d.t_fused_split_us
    assert abs(t - want) < 1e-9
    # head_dim 64 halves the streaming term
    lens = [1600] * 8
    two = pkv.pkv_policy_predict(lens, 8, CUS, pkv.PKV_MODE_SPLIT, 8, 1, head_dim=128)
    one = pkv.pkv_policy_predict(lens, 8, CUS, pkv.PKV_MODE_SPLIT, 8, 1, head_dim=64)
    fixed = d.t0_us + d.t_round_us + d.t_two_us + d.t_two_split_us * 8
    assert abs((two - fixed) - 2 * (one - fixed)) < 1e-9
    assert k["t_round_us"] == d.t_round_us
