"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the float64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from workloads import compact_rows

# Tolerance on fp16 outputs: max abs error <= 2e-3 and
# max abs error / max |reference| <= 1e-2, per case.
ATOL = 2e-3
RTOL = 1e-2
LSE_ATOL = 2e-3


def log_case(*parts):
    sys.stderr.write("[case] " + " ".join(str(p) for p in parts) + "\n")
    sys.stderr.flush()


def check_close(got, ref, atol=ATOL, rtol=RTOL, what="out"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert err <= atol, f"{what}: max abs err {err:.3e} > {atol}"
    if scale > 0:
        assert err / scale <= rtol, f"{what}: rel err {err / scale:.3e} > {rtol}"
    return err, (err / scale if scale > 0 else 0.0)


def check_lse(got, ref, atol=LSE_ATOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_r = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_r), "lse: -inf pattern differs"
    if (~inf_r).any():
        err = float(np.max(np.abs(got[~inf_r] - ref[~inf_r])))
        assert err <= atol, f"lse: max abs err {err:.3e}"


def run_hip(wl, mode=None, param=None, decoder=None, lse=True, repeats=1, two_launch=None,
            k_scale=1.0, v_scale=1.0):
    """Plan + decode through the C ABI (fused single launch, or the two-launch
    decode + merge form).  Returns (out tensor, lse tensor|None, decoder)."""
    import torch
    import paged_gqa_decode_pkv_amd as pkv

    cfg = wl.cfg
    if decoder is None:
        decoder = pkv.PagedDecoder(cfg.Hq, cfg.Hkv, cfg.D, max_batch=max(len(wl.seq_lens_np), 1),
                                   max_pages_per_row=wl.block_table_np.shape[1])
    out = torch.full_like(wl.q, float("nan"))
    lse_t = torch.full((wl.q.shape[0], cfg.Hq), float("nan"), dtype=torch.float32,
                       device=wl.q.device) if lse else None
    # host-side block-table check (what a serving loop does on admission)
    pkv.pkv_plan(wl.seq_lens_np, cfg.Hkv, wl.block_table_np.shape[1], 0, 1,
                 block_table=wl.block_table_np, num_pages=wl.k_pool.shape[0])
    decoder.set_inputs(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, wl.seq_lens_np,
                       cfg.scale, out, lse_t, k_scale=k_scale, v_scale=v_scale)
    for _ in range(repeats):
        decoder.run(mode, param, two_launch=two_launch)
    torch.cuda.synchronize()
    return out, lse_t, decoder


def check_bf16_rows(wl, got, got_lse, ref, ref_lse, rows=None, k_scale=1.0, v_scale=1.0,
                    where=""):
    """bf16 outputs (bf16 q; 2-byte or fp8 pools) against the oracle's ref /
    ref_lse on ``rows``: the rigorous elementwise and the statistical normwise
    bounds of tests/rounding_bound.py, with the softmax weights of the
    dequantised inputs.  Returns (max abs error, worst normwise ratio)."""
    from tests import rounding_bound
    if rows is None:
        rows = range(len(wl.seq_lens_np))
    q, k, v, bt, sl = compact_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, rows)
    stats = rounding_bound.softmax_stats(q, oracle.kv_values(k, k_scale), oracle.kv_values(v, v_scale),
                                     bt, sl, wl.cfg.scale * 1.0, ref)
    err, ratio = rounding_bound.check(got, got_lse, ref, ref_lse, stats, where)
    log_case("bf16 max abs err", f"{err:.3e}", "normwise / bound", f"{ratio:.3f}")
    return err, ratio


def oracle_rows(wl, rows=None, k_scale=1.0, v_scale=1.0):
    """Float64 oracle on the given rows (all rows by default), pages copied
    from wherever the workload lives (fp8 pools as their E4M3 codes)."""
    if rows is None:
        rows = range(len(wl.seq_lens_np))
    q, k, v, bt, sl = compact_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, rows)
    return oracle.attend(q, k, v, bt, sl, wl.cfg.scale, k_scale=k_scale, v_scale=v_scale)
