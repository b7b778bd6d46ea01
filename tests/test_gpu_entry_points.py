"""The one-shot entry points of the C ABI with caller-owned buffers, and the
runner's workspace handling across streams.

Every buffer here is a torch allocation made by the test (q, pools, table,
lengths, plan, outputs, workspace); the library only launches kernels on
them.  Results are compared with the float64 oracle (fp16 bar: max abs 2e-3,
max abs / max |ref| 1e-2) and, between launch forms, bit for bit.
"""
import numpy as np
import pytest

from tests.gpu_util import check_close, check_lse, log_case, oracle_rows, run_hip
from workloads import HELD_OUT_SEEDS, make_workload

pytestmark = pytest.mark.gpu

SEED = HELD_OUT_SEEDS[0]


def _caller_owned(wl, mode, param):
    """Host plan -> device tensors, workspace sized by pkv_workspace_size."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    cfg = wl.cfg
    tasks, offs, slots = pkv.pkv_plan(wl.seq_lens_np, cfg.Hkv, cfg.max_pages_per_row, mode, param,
                                      block_table=wl.block_table_np,
                                      num_pages=wl.k_pool.shape[0])
    t_d = torch.from_numpy(tasks).cuda()
    o_d = torch.from_numpy(offs).cuda()
    ws = torch.zeros(pkv.pkv_workspace_size(slots, cfg.Hq, cfg.D), dtype=torch.uint8,
                     device="cuda")
    pkv.pkv_workspace_init(ws)
    out = torch.full_like(wl.q, float("nan"))
    lse = torch.full((wl.q.shape[0], cfg.Hq), float("nan"), dtype=torch.float32, device="cuda")
    return t_d, o_d, slots, ws, out, lse


@pytest.mark.parametrize("name,mode,param", [("tiny", 0, 4), ("b1", 0, 32), ("b8_bimodal", 1, 128),
                                             ("b8_bimodal", 1, 16)])
def test_one_shot_entry_points(name, mode, param):
    """pkv_decode (merge fused), and pkv_decode_splits then pkv_merge, on
    caller-owned buffers: each matches the oracle, and the two give the same
    bits."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    log_case("one-shot", name, "mode", mode, "param", param)
    wl = make_workload(name, SEED, device="cuda")
    cfg = wl.cfg
    ref, ref_lse = oracle_rows(wl)
    t_d, o_d, slots, ws, out, lse = _caller_owned(wl, mode, param)
    pkv.pkv_decode(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, t_d, o_d, slots,
                   cfg.scale, out, ws, lse=lse)
    torch.cuda.synchronize()
    a, la = out.cpu().numpy().copy(), lse.cpu().numpy().copy()
    check_close(a.astype(np.float64), ref)
    check_lse(la, ref_lse)
    assert pkv.pkv_workspace_error_flags(ws) == 0
    t_d, o_d, slots, ws2, out2, lse2 = _caller_owned(wl, mode, param)
    pkv.pkv_decode_splits(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, t_d, o_d,
                          slots, cfg.scale, out2, ws2, lse=lse2)
    pkv.pkv_merge(o_d, slots, cfg.Hkv, out2, ws2, lse=lse2)
    torch.cuda.synchronize()
    assert np.array_equal(a, out2.cpu().numpy())
    assert np.array_equal(la, lse2.cpu().numpy())
    assert pkv.pkv_workspace_error_flags(ws2) == 0


@pytest.mark.parametrize("name", ["b1", "b8_bimodal"])
def test_plan_and_decode(name):
    """The plan() / decode() names: policy, plan and one step, both launch forms."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload(name, SEED, device="cuda")
    cfg = wl.cfg
    p = pkv.plan(wl.seq_lens_np, cfg.Hkv, cfg.max_pages_per_row, head_dim=cfg.D,
                 block_table=wl.block_table_np, num_pages=wl.k_pool.shape[0])
    assert p.mode == (pkv.PKV_MODE_SPLIT if name == "b1" else pkv.PKV_MODE_WORKQUEUE)
    ref, ref_lse = oracle_rows(wl)
    for two in (False, True):
        lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
        out, _ = pkv.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, p,
                            cfg.scale, lse=lse, two_launch=two)
        torch.cuda.synchronize()
        check_close(out.float().cpu().numpy(), ref)
        check_lse(lse.cpu().numpy(), ref_lse)


def test_runner_regrows_workspace_on_a_side_stream():
    """A step on a non-current stream whose plan needs a bigger workspace:
    the decoder waits for that stream before replacing the workspace; then
    steps alternate between streams (reading the runner's device copy of the
    plan on both) and every result equals that of a fresh decoder."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("b8_bimodal", SEED, device="cuda")
    cfg = wl.cfg
    fresh = {}
    for mode, param in ((1, 128), (1, 8)):
        o, l, _ = run_hip(wl, mode, param)
        fresh[(mode, param)] = (o.cpu().numpy(), l.cpu().numpy())
    dec = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=cfg.B,
                           max_pages_per_row=cfg.max_pages_per_row)
    small = dec.workspace.numel()
    out = torch.empty_like(wl.q)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
    dec.set_inputs(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, wl.seq_lens_np,
                   cfg.scale, out, lse)
    side = torch.cuda.Stream()
    steps = [(side, 1, 128), (side, 1, 128), (None, 1, 128), (side, 1, 8), (side, 1, 8),
             (None, 1, 8), (side, 1, 8), (None, 1, 128), (side, 1, 128)]
    for st, mode, param in steps:
        log_case("runner stream step", "side" if st is not None else "current", mode, param)
        dec.run(mode, param, stream=st)
        (st or torch.cuda.current_stream()).synchronize()
        assert np.array_equal(out.cpu().numpy(), fresh[(mode, param)][0])
        assert np.array_equal(lse.cpu().numpy(), fresh[(mode, param)][1])
    assert dec.workspace.numel() > small
    assert dec.error_flags() == 0


def test_runner_follows_the_current_stream():
    """With no stream argument a step runs on torch's current stream, found
    without building a Stream object: inside a side stream's context it is
    that stream, and the result matches a step on the default stream bit
    for bit."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    assert pkv.current_stream_ptr() == torch.cuda.current_stream().cuda_stream
    wl = make_workload("b8_bimodal", SEED, device="cuda")
    cfg = wl.cfg
    dec = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=cfg.B,
                           max_pages_per_row=cfg.max_pages_per_row)
    out = torch.empty_like(wl.q)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
    dec.set_inputs(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, wl.seq_lens_np,
                   cfg.scale, out, lse)
    log_case("runner current stream", "default")
    dec.run()
    torch.cuda.synchronize()
    ref_o, ref_l = out.cpu().numpy(), lse.cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert pkv.current_stream_ptr() == side.cuda_stream
        out.fill_(float("nan"))
        log_case("runner current stream", "side")
        for _ in range(3):
            dec.run()
    side.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref_o)
    assert np.array_equal(lse.cpu().numpy(), ref_l)
    assert pkv.current_stream_ptr() == torch.cuda.current_stream().cuda_stream
    assert dec.error_flags() == 0


def test_runner_plan_across_length_changes():
    """Steps whose lengths move within their last page keep the plan (the
    runner's device copy serves them); steps that cross a page boundary get a
    new one (read in place from pinned memory, then copied for the next
    steps).  Every step matches a fresh runner's bit for bit, in both launch
    forms."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("b8_bimodal", SEED, device="cuda")
    cfg = wl.cfg
    base = wl.seq_lens_np.astype(np.int32).copy()
    base[0] = max(1, (int(base[0]) - 2) // 16 * 16 + 1)    # a row one token into its last page
    within = base - (base % 16 != 1) * (base > 1)          # same page counts
    across = base - (base % 16 == 1)                        # fewer pages in some rows
    assert (across != base).any() and (within != base).any()
    seq_dev = torch.from_numpy(base.copy()).cuda()
    out = torch.empty_like(wl.q)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
    dec = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=cfg.B,
                           max_pages_per_row=cfg.max_pages_per_row)
    steps = [base, base, within, within, base, across, across, within, base]
    for two in (None, True):
        for i, lens in enumerate(steps):
            log_case("runner plan across lengths", i, "two" if two else "rule")
            seq_dev.copy_(torch.from_numpy(lens))
            dec.set_inputs(wl.q, wl.k_pool, wl.v_pool, wl.block_table, seq_dev, lens, cfg.scale,
                           out, lse)
            dec.run(two_launch=two)
            fresh = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=cfg.B,
                                     max_pages_per_row=cfg.max_pages_per_row)
            out2 = torch.empty_like(wl.q)
            lse2 = torch.empty_like(lse)
            fresh.set_inputs(wl.q, wl.k_pool, wl.v_pool, wl.block_table, seq_dev, lens,
                             cfg.scale, out2, lse2)
            fresh.run(two_launch=two)
            torch.cuda.synchronize()
            assert dec.last == fresh.last
            assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())
            assert np.array_equal(lse.cpu().numpy(), lse2.cpu().numpy())
            tasks, offs = dec.plan_arrays()
            t2, o2 = fresh.plan_arrays()
            assert np.array_equal(tasks, t2) and np.array_equal(offs, o2)
    assert dec.error_flags() == 0
