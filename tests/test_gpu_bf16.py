"""GPU parity with bfloat16 q, K, V and out (PKV_DTYPE_BF16).

The oracle is the same float64 definition, fed the exact float32 widening of
the bf16 inputs.  Tolerance, derived from the arithmetic (no value is given
for bf16):
  * the probabilities p = 2^(s - m) enter the PV product and the sum l as bf16,
    each with a relative error of at most 2^-9; a weighted average whose
    weights are each off by a factor (1 + d), |d| <= 2^-9, moves by at most
    2 * 2^-9 * max_t |v_t - out| <= 2^-8 * 2 max |v|;
  * the output is rounded once more to bf16: 2^-9 |out|.
  So per case: max abs err <= 2^-7 max|v| + 2^-9 max|ref|, with v the value
  entries the case attends to.  lse moves by at most log(1 + 2^-9) < 2^-8.
Scores and accumulators are fp32 from exact bf16 inputs, far below these.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import log_case, run_hip
from workloads import CALIBRATION_SEED, HELD_OUT_SEEDS, Config, compact_rows, make_workload

pytestmark = pytest.mark.gpu

SEED = HELD_OUT_SEEDS[0]


def _ref(wl, rows=None):
    if rows is None:
        rows = range(len(wl.seq_lens_np))
    q, k, v, bt, sl = compact_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, rows)
    out, lse = oracle.attend(q, k, v, bt, sl, wl.cfg.scale)
    vmax = float(np.nanmax(np.abs(v))) if v.size else 0.0
    return out, lse, vmax


def _check_bf16(got, got_lse, ref, ref_lse, vmax):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    bound = 2.0 ** -7 * vmax + 2.0 ** -9 * float(np.max(np.abs(ref)) if ref.size else 0.0)
    log_case("bf16 max abs err", f"{err:.3e}", "bound", f"{bound:.3e}")
    assert err <= bound, f"bf16 out: max abs err {err:.3e} > bound {bound:.3e}"
    inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), inf)
    if (~inf).any():
        lerr = float(np.max(np.abs(got_lse[~inf] - ref_lse[~inf])))
        assert lerr <= 2.0 ** -8, f"bf16 lse: max abs err {lerr:.3e}"
    return err, bound


def _parity(wl, mode=None, param=None, two_launch=None, rows=None):
    log_case("bf16", wl.cfg.name, "seed", wl.seed, "mode", mode, "param", param, "two", two_launch)
    out, lse, dec = run_hip(wl, mode, param, two_launch=two_launch)
    ref, ref_lse, vmax = _ref(wl, rows)
    sel = slice(None) if rows is None else list(rows)
    _check_bf16(out.float().cpu().numpy()[sel], lse.cpu().numpy()[sel], ref, ref_lse, vmax)
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
    ref, ref_lse, vmax = _ref(wl)
    _check_bf16(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, vmax)


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
