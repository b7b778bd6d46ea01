"""GPU parity with fp8 (OCP E4M3) K / V pools: PKV_DTYPE_F16_KV_FP8 and
PKV_DTYPE_BF16_KV_FP8.

The oracle decodes the pools' codes itself (``oracle.e4m3_decode``, from the
format's definition) and applies the per-tensor scales in float64.  Every
E4M3 value is exact in fp16 and in bf16, and the kernel converts the codes
exactly before the same MFMA path as the 2-byte pools, so the tolerances are
those of q's type: max abs 2e-3 and rel 1e-2 for fp16 q; for bf16 q the
bounds of tests/rounding_bound.py, with the softmax weights and values of the
dequantised pools.
"""
import numpy as np
import pytest

from tests.gpu_util import check_bf16_rows, check_close, check_lse, log_case, oracle_rows, run_hip
from workloads import CALIBRATION_SEED, HELD_OUT_SEEDS, Config, make_workload

pytestmark = pytest.mark.gpu

SEED = HELD_OUT_SEEDS[0]


def _parity(wl, mode=None, param=None, two_launch=None, k_scale=1.0, v_scale=1.0, rows=None):
    log_case("fp8", wl.cfg.name, "seed", wl.seed, "mode", mode, "param", param, "two",
             two_launch, "scales", k_scale, v_scale, "q", wl.q.dtype)
    out, lse, dec = run_hip(wl, mode, param, two_launch=two_launch, k_scale=k_scale,
                            v_scale=v_scale)
    ref, ref_lse = oracle_rows(wl, rows, k_scale=k_scale, v_scale=v_scale)
    sel = slice(None) if rows is None else list(rows)
    got = out.float().cpu().numpy()[sel]
    got_lse = lse.cpu().numpy()[sel]
    import torch
    if wl.q.dtype == torch.bfloat16:
        check_bf16_rows(wl, got, got_lse, ref, ref_lse, rows, k_scale, v_scale,
                        where=f"bf16 q fp8 pools {wl.cfg.name}")
    else:
        check_close(got, ref, atol=2e-3 * max(1.0, v_scale))   # out scales with v_scale
        check_lse(got_lse, ref_lse)
    assert dec.error_flags() == 0
    return out, lse


@pytest.mark.parametrize("name,mode,param", [("tiny", 0, 1), ("tiny", 0, 4), ("b1", 0, 32),
                                             ("b1", None, None), ("b8_bimodal", None, None),
                                             ("b8_bimodal", 1, 16), ("b8_zipf", None, None),
                                             ("b4_bimodal", None, None)])
@pytest.mark.parametrize("two_launch", [False, True])
def test_fp8_workloads(name, mode, param, two_launch):
    wl = make_workload(name, SEED, device="cuda", dtype="fp8")
    _parity(wl, mode, param, two_launch)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_ragged_gqa_ratios_and_head_dims(G, D):
    cfg = Config("small_fp8", B=0, Hq=G * 2, Hkv=2, D=D, max_pages_per_row=8, pool_pages=64,
                 lengths=lambda rng: np.zeros(0))
    lens = [1, 15, 16, 17, 33, 0, 127, 128]
    for mode, param in [(0, 1), (0, 3), (1, 1), (1, 2), (1, 8)]:
        wl = make_workload(cfg, 11 + G + D, device="cuda", seq_lens=lens, dtype="fp8")
        _parity(wl, mode, param)


@pytest.mark.parametrize("G", [1, 4, 16])
def test_fp8_head_dim_256(G):
    cfg = Config("small_fp8_d256", B=0, Hq=G * 2, Hkv=2, D=256, max_pages_per_row=8,
                 pool_pages=64, lengths=lambda rng: np.zeros(0))
    lens = [1, 15, 16, 17, 33, 0, 127, 128]
    for mode, param in [(0, 1), (0, 3), (1, 2), (1, 4)]:
        wl = make_workload(cfg, 13 + G, device="cuda", seq_lens=lens, dtype="fp8")
        _parity(wl, mode, param)


@pytest.mark.parametrize("k_scale,v_scale", [(0.5, 3.0), (2.0, 0.125)])
@pytest.mark.parametrize("two_launch", [False, True])
def test_fp8_dequantisation_scales(k_scale, v_scale, two_launch):
    wl = make_workload("b8_zipf", SEED, device="cuda", dtype="fp8")
    _parity(wl, 1, 64, two_launch, k_scale, v_scale)


def test_fp16_pools_with_unit_scales_are_unchanged():
    """With k_scale = v_scale = 1 the fp16 path is bit for bit the unscaled one,
    and non-unit scales on fp16 pools follow the oracle."""
    wl = make_workload("b8_bimodal", SEED, device="cuda")
    a, la, _ = run_hip(wl, 1, 64)
    b, lb, _ = run_hip(wl, 1, 64, k_scale=1.0, v_scale=1.0)
    assert np.array_equal(a.float().cpu().numpy(), b.float().cpu().numpy())
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy())
    _parity(wl, 1, 64, None, 0.75, 1.5)


@pytest.mark.parametrize("name", ["tiny", "b8_bimodal", "b1"])
def test_bf16_q_with_fp8_pools(name):
    wl = make_workload(name, SEED, device="cuda", dtype="bf16_fp8")
    _parity(wl)
    _parity(wl, 0, 4, True, 0.5, 2.0)


def test_fp8_fused_and_two_launch_agree():
    wl = make_workload("b8_bimodal", CALIBRATION_SEED, device="cuda", dtype="fp8")
    a, la, _ = run_hip(wl, 1, 8)
    b, lb, _ = run_hip(wl, 1, 8, two_launch=True)
    assert np.array_equal(a.float().cpu().numpy(), b.float().cpu().numpy())
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_fp8_poison_does_not_leak():
    """NaN codes in every unreferenced page and tail slot change nothing."""
    a = make_workload("b8_zipf", SEED, device="cuda", fill="nan", dtype="fp8")
    b = make_workload("b8_zipf", SEED, device="cuda", fill="random", dtype="fp8")
    oa, la, _ = run_hip(a, 1, 32)
    ob, lb, _ = run_hip(b, 1, 32)
    assert np.array_equal(oa.float().cpu().numpy(), ob.float().cpu().numpy())
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_fp8_device_planned_step():
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("b8_bimodal", SEED, device="cuda", dtype="fp8")
    cfg = wl.cfg
    need = pkv.pkv_workspace_size_device_plan(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, 64)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    pkv.pkv_workspace_init(ws)
    out = torch.empty_like(wl.q)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
    pkv.pkv_decode_device_plan(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, cfg.scale,
                               out, ws, 64, lse=lse, k_scale=0.5, v_scale=2.0)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_rows(wl, k_scale=0.5, v_scale=2.0)
    check_close(out.float().cpu().numpy(), ref)
    check_lse(lse.cpu().numpy(), ref_lse)
    assert pkv.pkv_workspace_error_flags(ws) == 0


def test_pool_types_checked():
    import torch
    import paged_gqa_decode_pkv_amd as pkv
    wl = make_workload("tiny", SEED, device="cuda", dtype="fp8")
    cfg = wl.cfg
    dec = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=1, max_pages_per_row=16)
    out = torch.empty_like(wl.q)
    with pytest.raises(TypeError):     # K fp8, V fp16
        dec.set_inputs(wl.q, wl.k_pool, wl.v_pool.view(torch.uint8).half(), wl.block_table,
                       wl.seq_lens, wl.seq_lens_np, cfg.scale, out)
    with pytest.raises(TypeError):     # pools as raw bytes
        dec.set_inputs(wl.q, wl.k_pool.view(torch.uint8), wl.v_pool.view(torch.uint8),
                       wl.block_table, wl.seq_lens, wl.seq_lens_np, cfg.scale, out)
    with pytest.raises(pkv.PkvError):  # scales must be > 0
        dec.set_inputs(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, wl.seq_lens_np,
                       cfg.scale, out, k_scale=0.0)
        dec.run()
