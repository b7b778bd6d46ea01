"""GPU parity with bfloat16 q, K, V and out (PKV_DTYPE_BF16).

The oracle is the same float64 definition, fed the exact widening of the
bf16 inputs.  The tolerance is derived from the kernel's arithmetic in
tests/rounding_bound.py: per (row, query head) a rigorous elementwise bound (the
probabilities enter PV and the sum as bf16, so the output moves by at most
u/(1-u) times their weighted spread sum_t w_t |v_t - out|, plus one output
rounding u |out|, u = 2^-8) and a statistical normwise bound (twice the RMS
of those roundings), which a dropped page, a wrong head map or a zeroed
output exceed at long context (shown on the CPU in tests/test_rounding_bound.py).
lse: within u/(1-u), and within 6 sigma of its rounding.
"""
import numpy as np
import pytest

from tests.gpu_util import check_bf16_rows, log_case, oracle_rows, run_hip
from workloads import CALIBRATION_SEED, HELD_OUT_SEEDS, Config, make_workload

pytestmark = pytest.mark.gpu

SEED = HELD_OUT_SEEDS[0]


def _parity(wl, mode=None, param=None, two_launch=None, rows=None):
    log_case("bf16", wl.cfg.name, "seed", wl.seed, "mode", mode, "param", param, "two", two_launch)
    out, lse, dec = run_hip(wl, mode, param, two_launch=two_launch)
    ref, ref_lse = oracle_rows(wl, rows)
    sel = slice(None) if rows is None else list(rows)
    check_bf16_rows(wl, out.float().cpu().numpy()[sel], lse.cpu().numpy()[sel], ref, ref_lse,
                    rows, where=f"bf16 {wl.cfg.name}")
    assert dec.error_flags() == 0
    return out, lse


@pytest.mark.parametrize("name,mode,param", [("tiny", 0, 1), ("tiny", 0, 4), ("b1", 0, 32),
                                             ("b1", None, None), ("b8_bimodal", None, None),
                                             ("b8_bimodal", 1, 16), ("b8_zipf", None, None),
                                             ("b4_bimodal", None, None)])
@pytest.mark.parametrize("two_launch", [False, True])
def test_bf16_workloads(name, mode, param, two_launch):
    wl = make_workload(name, SEED, device="cuda", dtype="bf16")
    _parity(wl, mode, param, two_launch)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_ragged_gqa_ratios_and_head_dims(G, D):
    cfg = Config("small_bf16", B=0, Hq=G * 2, Hkv=2, D=D, max_pages_per_row=8, pool_pages=64,
                 lengths=lambda rng: np.zeros(0))
    lens = [1, 15, 16, 17, 33, 0, 127, 128]
    for mode, param in [(0, 1), (0, 3), (1, 1), (1, 2)]:
        wl = make_workload(cfg, 5 + G + D, device="cuda", seq_lens=lens, dtype="bf16")
        _parity(wl, mode, param)


def test_bf16_fused_and_two_launch_agree():
    wl = make_workload("b8_bimodal", CALIBRATION_SEED, device="cuda", dtype="bf16")
    a, la, _ = run_hip(wl, 1, 8)
    b, lb, _ = run_hip(wl, 1, 8, two_launch=True)
    assert np.array_equal(a.float().cpu().numpy(), b.float().cpu().numpy())
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_bf16_poison_does_not_leak():
    a = make_workload("b8_zipf", SEED, device="cuda", fill="nan", dtype="bf16")
    b = make_workload("b8_zipf", SEED, device="cuda", fill="random", dtype="bf16")
    oa, la, _ = run_hip(a, 1, 32)
    ob, lb, _ = run_hip(b, 1, 32)
    assert np.array_equal(oa.float().cpu().numpy(), ob.float().cpu().numpy())
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_bf16_device_planned_step():
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("b8_bimodal", SEED, device="cuda", dtype="bf16")
    cfg = wl.cfg
    need = pkv.pkv_workspace_size_device_plan(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, 64)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    pkv.pkv_workspace_init(ws)
    out = torch.empty_like(wl.q)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
    pkv.pkv_decode_device_plan(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, cfg.scale,
                               out, ws, 64, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_rows(wl)
    check_bf16_rows(wl, out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse,
                    where="bf16 device plan")


def test_mixed_element_types_rejected():
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("tiny", SEED, device="cuda", dtype="bf16")
    cfg = wl.cfg
    dec = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=1, max_pages_per_row=16)
    with pytest.raises(TypeError):
        dec.set_inputs(wl.q, wl.k_pool.half(), wl.v_pool, wl.block_table, wl.seq_lens,
                       wl.seq_lens_np, cfg.scale, torch.empty_like(wl.q))


@pytest.mark.parametrize("G", [1, 4, 16])
def test_bf16_head_dim_256(G):
    cfg = Config("small_bf16_d256", B=0, Hq=G * 2, Hkv=2, D=256, max_pages_per_row=8,
                 pool_pages=64, lengths=lambda rng: np.zeros(0))
    lens = [1, 15, 16, 17, 33, 0, 127, 128]
    for mode, param in [(0, 1), (0, 3), (1, 2)]:
        wl = make_workload(cfg, 9 + G, device="cuda", seq_lens=lens, dtype="bf16")
        _parity(wl, mode, param)
