"""Randomised GPU parity: many small seeded cases across every supported shape,
element type, schedule and launch form, each against the float64 oracle.

Each case draws G, d, Hkv, B, the row lengths (including empty rows, single
tokens, page-boundary lengths and rows at the table width), the pool type,
the schedule (split S or workqueue c), the launch form and, for fp8 pools,
the dequantisation scales.  The bar is that of the element type (see
test_gpu_parity.py and tests/rounding_bound.py); with v_scale > 1
the absolute fp16 bound is 2e-3 * v_scale, since out and its rounding error
both scale with v_scale.
"""
import numpy as np
import pytest

from tests.gpu_util import check_bf16_rows, check_close, check_lse, log_case, oracle_rows, run_hip
from workloads import Config, make_workload

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 13))
    maxp = int(rng.choice([1, 3, 8, 33]))
    special = [x for x in (0, 1, 15, 16, 17, 16 * maxp, 16 * maxp - 1) if x <= 16 * maxp]
    lens = [int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(0, 16 * maxp + 1))
            for _ in range(B)]
    dtype = str(rng.choice(["f16", "bf16", "fp8", "bf16_fp8"]))
    mode = int(rng.integers(0, 2))
    param = int(rng.choice([1, 2, 3, 4, 7, 16])) if mode == 0 else int(rng.choice([1, 2, 4, 5, 8]))
    two = bool(rng.integers(0, 2))
    fill = str(rng.choice(["nan", "random"]))
    scales = (1.0, 1.0)
    if dtype.endswith("fp8") and rng.random() < 0.5:
        scales = (float(rng.choice([0.25, 0.5, 2.0])), float(rng.choice([0.5, 1.5, 4.0])))
    return G, D, Hkv, B, maxp, lens, dtype, mode, param, two, fill, scales


@pytest.mark.parametrize("seed", range(150))
def test_random_case(seed):
    import torch
    G, D, Hkv, B, maxp, lens, dtype, mode, param, two, fill, (ks, vs) = _case(seed)
    log_case("random", seed, "G", G, "D", D, "Hkv", Hkv, "lens", lens, "dtype", dtype, "mode", mode,
             "param", param, "two", two, "fill", fill, "scales", ks, vs)
    cfg = Config(f"rand{seed}", B=0, Hq=G * Hkv, Hkv=Hkv, D=D, max_pages_per_row=maxp,
                 pool_pages=B * maxp + 5, lengths=lambda r: np.zeros(0))
    wl = make_workload(cfg, 1000 + seed, device="cuda", seq_lens=lens, fill=fill, dtype=dtype)
    out, lse, dec = run_hip(wl, mode, param, two_launch=two, k_scale=ks, v_scale=vs)
    ref, ref_lse = oracle_rows(wl, k_scale=ks, v_scale=vs)
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    if wl.q.dtype == torch.bfloat16:
        check_bf16_rows(wl, got, got_lse, ref, ref_lse, None, ks, vs, where=f"random {seed}")
    else:
        # out is linear in v_scale, and so is its rounding error: the absolute
        # bound scales with it (the relative one does not change)
        check_close(got, ref, atol=2e-3 * max(1.0, vs))
        check_lse(got_lse, ref_lse)
    assert dec.error_flags() == 0
