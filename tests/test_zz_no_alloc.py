"""pkv_decode_static, the entry point that allocates nothing, against
pkv_decode on the same inputs and plan: bit for bit, on two calls in a row
(the second a smaller step), through the C ABI; and its size limit."""
import numpy as np
import pytest

from tests.gpu_util import log_case
from workloads import HELD_OUT_SEEDS, make_workload

pytestmark = pytest.mark.gpu


def _inputs(name, mode, param):
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload(name, HELD_OUT_SEEDS[0], device="cuda")
    cfg = wl.cfg
    tasks, offs, slots = pkv.pkv_plan(wl.seq_lens_np, cfg.Hkv, cfg.max_pages_per_row, mode, param,
                                      block_table=wl.block_table_np,
                                      num_pages=wl.k_pool.shape[0])
    return wl, torch.from_numpy(tasks).cuda(), torch.from_numpy(offs).cuda(), slots


def test_no_alloc_entry_point_matches_pkv_decode():
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    for name, mode, param in (("b8_bimodal", 1, 128), ("tiny", 0, 4)):
        log_case("no-alloc", name, mode, param)
        wl, t_d, o_d, slots = _inputs(name, mode, param)
        cfg = wl.cfg
        ws = torch.zeros(pkv.pkv_workspace_size(slots, cfg.Hq, cfg.D), dtype=torch.uint8,
                         device="cuda")
        pkv.pkv_workspace_init(ws)
        out_a = torch.full_like(wl.q, float("nan"))
        lse_a = torch.full((cfg.B, cfg.Hq), float("nan"), dtype=torch.float32, device="cuda")
        pkv.pkv_decode(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, t_d, o_d, slots,
                       cfg.scale, out_a, ws, lse=lse_a)
        out_b = torch.full_like(wl.q, float("nan"))
        lse_b = torch.full((cfg.B, cfg.Hq), float("nan"), dtype=torch.float32, device="cuda")
        pkv.pkv_decode_static(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, t_d, o_d,
                              slots, cfg.scale, out_b, lse=lse_b)
        torch.cuda.synchronize()
        assert np.array_equal(out_a.cpu().numpy(), out_b.cpu().numpy())
        assert np.array_equal(lse_a.cpu().numpy(), lse_b.cpu().numpy())
        assert np.all(np.isfinite(out_b.float().cpu().numpy()))


def test_no_alloc_entry_point_rejects_oversize_steps():
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl, t_d, o_d, slots = _inputs("tiny", 0, 4)
    cfg = wl.cfg
    out = torch.empty_like(wl.q)
    big = (pkv.PKV_STATIC_SCRATCH_BYTES // (cfg.Hq * (cfg.D + 2) * 4)) + 1
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_static(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, t_d, o_d,
                              big, cfg.scale, out)
    assert e.value.status == pkv.PKV_ERR_SCRATCH_TOO_SMALL
