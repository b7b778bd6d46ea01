"""GPU: the device-side planner (pkv_decode_device_plan).

The plan the planner kernel writes must equal the host planner's, bit for bit,
and the policy it evaluates on the device must take the host policy's
decision (both limited to the capacity).  The outputs are checked against the
float64 oracle like every other schedule.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import check_close, check_lse, log_case, oracle_rows
from workloads import CALIBRATION_SEED, CONFIGS, HELD_OUT_SEEDS, Config, make_workload

pytestmark = pytest.mark.gpu

SEED = HELD_OUT_SEEDS[0]


def _capped_params(pkv, max_pages, cap, groups):
    """The host policy's candidate sets limited the way the device path limits
    them; with the groups within the fused merge's counters, the launch-form
    rule off (the device-planned step is always fused)."""
    p = pkv.pkv_policy_defaults()
    if groups <= pkv.PKV_MAX_FUSED_GROUPS:
        p.fuse_max_splits = 2 ** 31 - 1
    p.split_max = min(p.split_max, cap)
    c = p.chunk_min
    while c <= p.chunk_max and -(-max_pages // c) > cap:
        c *= 2
    p.chunk_min = c
    return p


def _run(wl, cap, mode=-1, param=0, workspace=None, params=None):
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    cfg = wl.cfg
    B = len(wl.seq_lens_np)
    need = pkv.pkv_workspace_size_device_plan(B, cfg.Hq, cfg.Hkv, cfg.D, cap)
    if workspace is None or workspace.numel() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device="cuda")
        pkv.pkv_workspace_init(workspace)
    out = torch.full_like(wl.q, float("nan"))
    lse = torch.full((B, cfg.Hq), float("nan"), dtype=torch.float32, device="cuda")
    pkv.pkv_decode_device_plan(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, cfg.scale,
                               out, workspace, cap, lse=lse, mode=mode, param=param,
                               params=params)
    torch.cuda.synchronize()
    hdr, tasks, offs = pkv.pkv_device_plan_read(workspace, B, cfg.Hq, cfg.Hkv, cfg.D, cap)
    return out, lse, hdr, tasks, offs, workspace


def _check_plan(wl, cap, hdr, tasks, offs, mode, param):
    import paged_gqa_decode_pkv_amd as pkv
    cfg = wl.cfg
    maxp = wl.block_table_np.shape[1]
    if mode < 0:
        p = _capped_params(pkv, maxp, cap, len(wl.seq_lens_np) * cfg.Hkv)
        if p.chunk_min <= p.chunk_max:
            want = pkv.pkv_policy(wl.seq_lens_np, cfg.Hkv, _num_cus(), params=p, head_dim=cfg.D)
        else:
            # no workqueue schedule fits: the first fastest split candidate
            # (timed with valid chunk bounds; the model does not read them)
            p.chunk_min = p.chunk_max
            best = None
            S = 1
            while S <= p.split_max:
                t = pkv.pkv_policy_predict(wl.seq_lens_np, cfg.Hkv, _num_cus(), 0, S,
                                           params=p, head_dim=cfg.D)
                if best is None or t < best[0]:
                    best = (t, (0, S))
                S *= 2
            want = best[1]
        assert (hdr["mode"], hdr["param"]) == want
        mode, param = want
    assert (hdr["mode"], hdr["param"]) == (mode, param)
    rt, ro, slots = pkv.pkv_plan(wl.seq_lens_np, cfg.Hkv, maxp, mode, param)
    assert np.array_equal(tasks, rt)
    assert np.array_equal(offs, ro)
    assert hdr["num_tasks"] == len(rt) and hdr["num_partial_slots"] == slots
    deepest = int(np.max(np.diff(ro))) if len(ro) > 1 else 0
    assert hdr["max_splits"] == deepest
    groups = cfg.Hkv * len(wl.seq_lens_np)
    assert hdr["fused"] == int(len(rt) == 0 or groups <= pkv.PKV_MAX_FUSED_GROUPS)
    assert hdr["row_flagged"] == 0


def _num_cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _parity(wl, out, lse, rows=None):
    ref_out, ref_lse = oracle_rows(wl, rows)
    sel = slice(None) if rows is None else list(rows)
    check_close(out.float().cpu().numpy()[sel], ref_out)
    check_lse(lse.cpu().numpy()[sel], ref_lse)


@pytest.mark.parametrize("name", ["tiny", "b1", "b1_bucketed", "b4_bimodal", "b8_bimodal",
                                  "b8_zipf", "b8_uniform"])
def test_device_policy_plan_and_parity(name):
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload(name, SEED, device="cuda")
    log_case("device plan", name, "seed", SEED)
    out, lse, hdr, tasks, offs, ws = _run(wl, cap=256)
    _check_plan(wl, 256, hdr, tasks, offs, -1, 0)
    _parity(wl, out, lse)
    assert pkv.pkv_workspace_error_flags(ws) == 0


@pytest.mark.parametrize("mode,param", [(0, 1), (0, 8), (0, 64), (1, 4), (1, 32), (1, 256)])
def test_device_plan_explicit_schedules(mode, param):
    wl = make_workload("b8_bimodal", CALIBRATION_SEED, device="cuda")
    cap = 256
    log_case("device plan explicit", mode, param)
    out, lse, hdr, tasks, offs, _ = _run(wl, cap, mode, param)
    _check_plan(wl, cap, hdr, tasks, offs, mode, param)
    _parity(wl, out, lse)


def test_device_policy_under_a_small_capacity():
    """max_splits = 4: the device policy only sees schedules that fit, and
    takes the host policy's decision over the same limited candidates."""
    wl = make_workload("b1", SEED, device="cuda")
    out, lse, hdr, tasks, offs, _ = _run(wl, cap=4)
    _check_plan(wl, 4, hdr, tasks, offs, -1, 0)
    assert hdr["max_splits"] <= 4
    _parity(wl, out, lse)


@pytest.mark.parametrize("kind", ["workqueue", "split"])
def test_device_policy_over_several_candidate_batches(kind):
    """More than 16 candidates (the device search takes 16 per barrier): 21
    chunk sizes c = 1 .. 2^20 for a batch, or 18 split counts S = 1 .. 2^17
    for one row.  The device picks what the host policy picks under the same
    constants, limits and launch form, and the step matches the oracle."""
    import paged_gqa_decode_pkv_amd as pkv
    rng = np.random.default_rng(41 if kind == "workqueue" else 42)
    if kind == "workqueue":
        lens = rng.integers(1, 64 * 16 + 1, size=6).tolist()
        cap = 64
    else:
        lens = [int(rng.integers(200, 64 * 16 + 1))]
        cap = 1 << 17
    cfg = Config(f"multibatch_{kind}", B=len(lens), Hq=8, Hkv=2, D=64, max_pages_per_row=64,
                 pool_pages=len(lens) * 64 + 8, lengths=None)
    wl = make_workload(cfg, 43, device="cuda", seq_lens=lens)
    log_case("device policy, several candidate batches", kind, lens)
    p = pkv.pkv_policy_defaults()
    p.split_max = 1 << 20
    p.chunk_min = 1
    p.chunk_max = 1 << 20
    out, lse, hdr, tasks, offs, _ = _run(wl, cap, params=p)
    # the host policy under the device path's limits and launch form
    q = pkv.pkv_policy_defaults()
    q.split_max = min(p.split_max, cap)
    c = p.chunk_min
    while c <= p.chunk_max and -(-64 // c) > cap:
        c *= 2
    q.chunk_min, q.chunk_max = c, p.chunk_max
    q.fuse_max_splits = 2 ** 31 - 1
    ncand = (q.split_max.bit_length() if kind == "split"
             else (q.chunk_max // q.chunk_min).bit_length())
    assert ncand > 16
    want = pkv.pkv_policy(wl.seq_lens_np, cfg.Hkv, _num_cus(), params=q, head_dim=cfg.D)
    assert (hdr["mode"], hdr["param"]) == want
    assert hdr["mode"] == (0 if kind == "split" else 1)
    rt, ro, slots = pkv.pkv_plan(wl.seq_lens_np, cfg.Hkv, 64, *want)
    assert np.array_equal(tasks, rt) and np.array_equal(offs, ro)
    _parity(wl, out, lse)


@pytest.mark.parametrize("G,D", [(1, 64), (2, 128), (8, 128), (4, 64)])
def test_device_plan_ragged_edge_rows(G, D):
    lens = [1, 15, 16, 17, 33, 0, 127, 128, 4000, 0]
    cfg = Config(f"ragged_dp_G{G}_d{D}", B=len(lens), Hq=2 * G, Hkv=2, D=D,
                 max_pages_per_row=256, pool_pages=600, lengths=None)
    wl = make_workload(cfg, SEED, device="cuda", seq_lens=lens)
    log_case("device plan ragged", G, D)
    out, lse, hdr, tasks, offs, _ = _run(wl, cap=64)
    _check_plan(wl, 64, hdr, tasks, offs, -1, 0)
    _parity(wl, out, lse)


def test_device_plan_all_rows_empty():
    import torch
    lens = [0, 0, 0]
    cfg = Config("empty_dp", B=3, Hq=8, Hkv=2, D=128, max_pages_per_row=4, pool_pages=16,
                 lengths=None)
    wl = make_workload(cfg, SEED, device="cuda", seq_lens=lens)
    out, lse, hdr, tasks, offs, _ = _run(wl, cap=8)
    assert hdr["num_tasks"] == 0 and hdr["fused"] == 1
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_device_plan_reused_workspace_new_lengths():
    """One workspace, steps with different device lengths (and so different
    plans and policy choices): every step matches the oracle."""
    ws = None
    for seed in HELD_OUT_SEEDS[:3]:
        for name in ("b8_bimodal", "b4_bimodal"):
            wl = make_workload(name, seed, device="cuda")
            log_case("device plan reuse", name, seed)
            out, lse, hdr, tasks, offs, ws = _run(wl, cap=256, workspace=ws)
            _check_plan(wl, 256, hdr, tasks, offs, -1, 0)
            _parity(wl, out, lse)


def test_device_plan_kept_decision_follows_lengths_and_limits():
    """A self-planned step keeps its policy decision in the plan header for the
    next step on the workspace, keyed by the batch's page counts, shape and
    policy limits.  Steps that repeat a batch, change it, or change the
    capacity (and so the candidate sets) each take the host policy's decision
    under their own limits."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wls = {s: make_workload("b8_bimodal", s, device="cuda") for s in HELD_OUT_SEEDS[:2]}
    cfg = wls[HELD_OUT_SEEDS[0]].cfg
    need = pkv.pkv_workspace_size_device_plan(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, 256)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    pkv.pkv_workspace_init(ws)
    steps = [(0, 256), (0, 256), (1, 256), (1, 4), (1, 4), (0, 4), (0, 256), (1, 256)]
    for w, cap in steps:
        wl = wls[HELD_OUT_SEEDS[w]]
        log_case("kept decision", "seed", wl.seed, "cap", cap)
        out, lse, hdr, tasks, offs, _ = _run(wl, cap=cap, workspace=ws)
        _check_plan(wl, cap, hdr, tasks, offs, -1, 0)
        _parity(wl, out, lse)


def test_device_plan_ignores_a_corrupt_kept_decision():
    """Garbage in the kept-decision words of the plan header (a torn write, a
    stale workspace) never reaches the plan: each step still takes the host
    policy's decision and matches the oracle, bit for bit with a clean run."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("b1", SEED, device="cuda")
    cfg = wl.cfg
    B = len(wl.seq_lens_np)
    cap = 64
    plan_off = pkv.pkv_workspace_size(B * cap, cfg.Hq, cfg.D)
    ref_out, ref_lse, hdr0, tasks0, offs0, ws = _run(wl, cap=cap)
    _check_plan(wl, cap, hdr0, tasks0, offs0, -1, 0)
    rng = np.random.default_rng(7)
    words = ws[plan_off:plan_off + 64].view(torch.int32)
    kept = words[8:12].clone()
    trials = [rng.integers(-2 ** 31, 2 ** 31, size=4, dtype=np.int64) for _ in range(4)]
    trials.append(np.zeros(4, dtype=np.int64))
    good = kept.cpu().numpy().astype(np.int64)
    for k in range(4):           # the kept entry with one word changed
        t = good.copy()
        t[k] ^= 1 << (5 + 7 * k)
        trials.append(t)
    for t in trials:
        log_case("corrupt kept decision", t.tolist())
        words[8:12] = torch.tensor(t.astype(np.int32), device="cuda")
        torch.cuda.synchronize()
        out, lse, hdr, tasks, offs, _ = _run(wl, cap=cap, workspace=ws)
        _check_plan(wl, cap, hdr, tasks, offs, -1, 0)
        assert np.array_equal(out.cpu().numpy(), ref_out.cpu().numpy())
        assert np.array_equal(lse.cpu().numpy(), ref_lse.cpu().numpy())


def test_device_plan_flags_overlong_row_and_plans_it_empty():
    """A length beyond max_pages_per_row * 16 is caught by the planner's own
    bounds check: that row comes out empty and the error word is set; the
    other rows are exact."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    lens = [100, 300, 50]
    cfg = Config("overlong_dp", B=3, Hq=8, Hkv=2, D=128, max_pages_per_row=32, pool_pages=128,
                 lengths=None)
    wl = make_workload(cfg, SEED, device="cuda", seq_lens=lens)
    bad = wl.seq_lens.clone()
    bad[1] = 32 * 16 + 1                      # one token past the table
    B = 3
    need = pkv.pkv_workspace_size_device_plan(B, cfg.Hq, cfg.Hkv, cfg.D, 8)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    pkv.pkv_workspace_init(ws)
    out = torch.full_like(wl.q, float("nan"))
    lse = torch.full((B, cfg.Hq), float("nan"), dtype=torch.float32, device="cuda")
    pkv.pkv_decode_device_plan(wl.q, wl.k_pool, wl.v_pool, wl.block_table, bad, cfg.scale, out,
                               ws, 8, lse=lse)
    torch.cuda.synchronize()
    hdr, _, offs = pkv.pkv_device_plan_read(ws, B, cfg.Hq, cfg.Hkv, cfg.D, 8)
    assert hdr["row_flagged"] == 1 and offs[2] - offs[1] == 0
    assert pkv.pkv_workspace_error_flags(ws) & pkv.PKV_DEVERR_ROW
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))
    _parity(wl, out, lse, rows=[0, 2])


def test_device_plan_step_in_a_graph_follows_new_lengths():
    """The device-planned step needs nothing from the host, so it can be
    captured once in a graph and replayed while the lengths in device memory
    change: every replay equals the eager step on the same lengths, bit for
    bit, and the oracle."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("b8_bimodal", SEED, device="cuda")
    cfg = wl.cfg
    B, cap = cfg.B, 64
    need = pkv.pkv_workspace_size_device_plan(B, cfg.Hq, cfg.Hkv, cfg.D, cap)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    pkv.pkv_workspace_init(ws)
    lens_dev = wl.seq_lens.clone()
    out = torch.empty_like(wl.q)
    lse = torch.empty((B, cfg.Hq), dtype=torch.float32, device="cuda")

    def step():
        pkv.pkv_decode_device_plan(wl.q, wl.k_pool, wl.v_pool, wl.block_table, lens_dev,
                                   cfg.scale, out, ws, cap, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    base = wl.seq_lens_np.astype(np.int64)
    for rep in range(4):
        # shorter rows only: their pages are already in the block table
        new = np.maximum(base - rng.integers(0, 3000, size=B), 0).astype(np.int32)
        if rep == 3:
            new[:] = 0
        lens_dev.copy_(torch.from_numpy(new).cuda())
        torch.cuda.synchronize()
        log_case("graph replay", rep, new.tolist())
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got, got_lse = out.clone(), lse.clone()
        out.fill_(float("nan"))
        step()                                    # eager, same lengths
        torch.cuda.synchronize()
        assert torch.equal(got, out) and torch.equal(got_lse, lse)
        wl_new = _with_lengths(wl, new)
        ref_out, ref_lse = oracle_rows(wl_new)
        check_close(got.float().cpu().numpy(), ref_out)
        check_lse(got_lse.cpu().numpy(), ref_lse)
    assert pkv.pkv_workspace_error_flags(ws) == 0


def _with_lengths(wl, lens):
    """The same pages and table, shorter lengths (for the oracle)."""
    import dataclasses
    import torch
    return dataclasses.replace(wl, seq_lens_np=np.asarray(lens, dtype=np.int32),
                               seq_lens=torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda())


def test_device_plan_head_dim_256():
    cfg = Config("d256_dp", B=8, Hq=16, Hkv=4, D=256, max_pages_per_row=1024,
                 pool_pages=2 * 8 * 1024, lengths=CONFIGS["b8_bimodal"].lengths)
    wl = make_workload(cfg, SEED, device="cuda")
    out, lse, hdr, tasks, offs, _ = _run(wl, cap=256)
    _check_plan(wl, 256, hdr, tasks, offs, -1, 0)
    _parity(wl, out, lse)


def test_device_plan_batch_beyond_lds_staging():
    rng = np.random.default_rng(32)
    B = 1100
    lens = rng.integers(0, 300, size=B)
    cfg = Config("b1100_dp", B=B, Hq=8, Hkv=2, D=64, max_pages_per_row=19,
                 pool_pages=B * 19 + 64, lengths=None)
    wl = make_workload(cfg, 32, device="cuda", seq_lens=lens.tolist())
    out, lse, hdr, tasks, offs, _ = _run(wl, cap=8)
    _check_plan(wl, 8, hdr, tasks, offs, -1, 0)
    rows = sorted(rng.choice(B, size=48, replace=False).tolist())
    _parity(wl, out, lse, rows=rows)


@pytest.mark.parametrize("name,dtype,mode,param", [
    ("b8_zipf", "f16", 1, 256),       # 208 tasks: both steps stream V with nt
    ("b8_bimodal", "f16", 1, 128),    # 256 tasks: likewise
    ("b32_uniform", "f16", 1, 128),   # 2472 tasks: the host step streams K and V with nt
    ("b8_zipf", "fp8", 1, 256),
])
def test_device_step_equals_host_step_bit_for_bit(name, dtype, mode, param):
    """The same plan computes the same bits whichever way it was planned and
    whatever cache policy its page loads carry: the device-planned step streams
    the V loads with nt; the host-planned step streams K too when a 2-byte
    pool's plan has more tasks than twice the CUs."""
    from tests.gpu_util import run_hip
    wl = make_workload(name, SEED, device="cuda", dtype=dtype)
    log_case("device vs host step", name, dtype, mode, param)
    host_out, host_lse, dec = run_hip(wl, mode, param)
    assert dec.last[:2] == (mode, param) and not dec.last[5]
    out, lse, hdr, _, _, _ = _run(wl, 256, mode, param)
    assert hdr["fused"] == 1
    assert np.array_equal(out.float().cpu().numpy(), host_out.float().cpu().numpy())
    assert np.array_equal(lse.cpu().numpy(), host_lse.cpu().numpy())
