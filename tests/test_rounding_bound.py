"""The tolerances of tests/rounding_bound.py can fail (CPU only).

At the long-context shapes (B1, N = 32768; B8 bimodal) the bound must
* accept an emulation of the kernel's bf16 rounding (p_t rounded to bf16 in
  numerator and denominator, output rounded to bf16), and
* reject a zeroed output, the head map h mod Hkv, and one dropped page of one
  row (all KV heads), each rounded to bf16 as a kernel would write it.
At fp16 (unit roundoff 2^-11) an emulation of the kernel's rounding must sit
well inside the statistical bound too, since the GPU tests compare schedules
with it.  The emulation and the mistakes are test code, on the CPU.
"""
import math

import numpy as np
import pytest

import oracle
from tests import rounding_bound
from workloads import compact_rows, make_workload


def _bf16(x):
    """Round to the nearest bfloat16 (ties to even), via float32."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(a.shape).astype(np.float64)


def _fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _attend(q, k, v, bt, sl, scale, head_map=None, drop=None, round_p=False, rnd=None):
    """float64 attention with the kernel's bf16 rounding of p (round_p), a
    head map other than floor(h/G), or one logical page (row, page) left out."""
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        N = int(sl[b])
        if N == 0:
            continue
        t = np.arange(N)
        if drop is not None and drop[0] == b:
            t = t[t // 16 != drop[1]]
        pages = bt[b, t // 16].astype(np.int64)
        slots = t % 16
        for h in range(Hq):
            g = head_map(h, Hkv, G) if head_map else h // G
            K = k[pages, g, slots, :]
            V = v[pages, g, slots, :]
            s = scale * (K @ q[b, h])
            m = s.max()
            p = np.exp(s - m)
            if round_p:
                p = (rnd or _bf16)(p)
            L = p.sum()
            out[b, h] = (p @ V) / L
            lse[b, h] = m + math.log(L)
    return out, lse


@pytest.fixture(scope="module", params=["b1", "b8_bimodal"])
def case(request):
    wl = make_workload(request.param, 20260623, device="cpu", fill="zero")
    rows = range(len(wl.seq_lens_np))
    q, k, v, bt, sl = compact_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, rows)
    q, k, v = _bf16(q), _bf16(k), _bf16(v)          # bf16 inputs, held exactly in float64
    scale = wl.cfg.scale
    ref, ref_lse = oracle.attend(q, k, v, bt, sl, scale)
    stats = rounding_bound.softmax_stats(q, k, v, bt, sl, scale, ref)
    return request.param, (q, k, v, bt, sl, scale), ref, ref_lse, stats


def test_emulated_kernel_rounding_passes(case):
    name, args, ref, ref_lse, stats = case
    out, lse = _attend(*args, round_p=True)
    err, ratio = rounding_bound.check(_bf16(out), lse, ref, ref_lse, stats, name)
    assert ratio < 0.8, (name, ratio)       # well inside the statistical bound


@pytest.mark.parametrize("mistake", ["zero", "head_mod", "dropped_page"])
def test_planted_mistakes_fail(case, mistake):
    name, args, ref, ref_lse, stats = case
    q, k, v, bt, sl, scale = args
    if mistake == "zero":
        out, lse = np.zeros_like(ref), ref_lse
    elif mistake == "head_mod":
        out, lse = _attend(*args, head_map=lambda h, Hkv, G: h % Hkv, round_p=True)
    else:
        b = int(np.argmax(sl))                          # the longest row, a middle page
        out, lse = _attend(*args, drop=(b, int(sl[b]) // 32), round_p=True)
    with pytest.raises(AssertionError):
        rounding_bound.check(_bf16(out), lse, ref, ref_lse, stats, f"{name} {mistake}")


def test_fp16_emulated_rounding_within_bound():
    wl = make_workload("b1", 20260622, device="cpu", fill="zero")
    q, k, v, bt, sl = compact_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.seq_lens, [0])
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    ref, ref_lse = oracle.attend(q, k, v, bt, sl, wl.cfg.scale)
    stats = rounding_bound.softmax_stats(q, k, v, bt, sl, wl.cfg.scale, ref)
    out, lse = _attend(q, k, v, bt, sl, wl.cfg.scale, round_p=True, rnd=_fp16)
    _, ratio = rounding_bound.check(_fp16(out), lse, ref, ref_lse, stats, "fp16",
                                    u=rounding_bound.U_FP16)
    assert ratio < 0.8, ratio
    # and a second realisation (p rounded at another scale, as a split with
    # another reference maximum rounds other values) stays within the
    # pairwise bound
    out2, _ = _attend(q * 1.0, k, v, bt, sl, wl.cfg.scale, round_p=True,
                      rnd=lambda p: _fp16(p * 3.0) / 3.0)
    rounding_bound.check_pair(_fp16(out), _fp16(out2), ref, stats, "fp16 pair")
