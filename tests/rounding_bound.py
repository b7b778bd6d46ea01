"""Error bounds for outputs of the decode kernel, derived from its
arithmetic (test infrastructure).  Used for bfloat16 outputs (no tolerance is
fixed for bf16, which the pages do not use) and for comparing fp16 results of
different schedules; the fp16 parity bar itself is the stated 2e-3 / 1e-2.

What the kernel computes: scores in fp32 from exact products of q and K
elements; p_t = 2^(s_t - m) for a reference m, rounded to q's type (unit
roundoff u: 2^-8 for bf16, 2^-11 for fp16) before it enters both the PV
product and the running sum l; fp32 accumulation; out = round(o / l) to
nearest even in q's type (unit roundoff u again); lse = m + log l.  Let w_t
be the exact softmax weights, out* the exact result, and delta_t the
relative rounding error of p_t (|delta_t| <= u).  The same rounded p_t sits
in numerator and denominator, so the exact-arithmetic result of the rounded
weights is

    o / l - out* = sum_t w_t delta_t (v_t - out*) / (1 + sum_t w_t delta_t).

Two checks per (row, query head), both from this identity:

* rigorous, element by element: |e_d| <= u/(1-u) * sum_t w_t |v_t,d - out*_d|
  plus the output rounding u |out*_d| (1 + u), with 2% and 1e-7 of slack for
  the fp32 score and accumulation errors (relative ~1e-5 at d <= 256).  This
  can never fail for a correct kernel, but at long context it admits the
  error of a few dropped pages, since it sums the worst case over all N
  tokens.

* statistical, normwise: round-to-nearest errors of unrelated values behave
  as independent zero-mean errors of variance at most u^2/3 (uniform within
  half an ulp), so E||e||^2 <= (u^2/3) (sum_t w_t^2 ||v_t - out*||^2 +
  ||out*||^2) (the second term is the output rounding).  The norm over d
  concentrates tightly (d >= 64 near-independent terms), so twice that RMS
  is never reached by a correct kernel, while a dropped page, a wrong head
  map or a zeroed output exceed it by a wide margin at bf16 (checked on the
  CPU in tests/test_rounding_bound.py, against an emulation of the kernel's
  rounding).
  lse:  lse - lse* = log(1 + sum_t w_t delta_t), RMS <= (u/sqrt 3) sqrt(sum_t
  w_t^2); a single value, so a 6-sigma band plus fp32 slack; the rigorous
  bound u/(1-u) is checked too.

Two results of the same inputs under different schedules (split counts,
launch forms) round different p values (each split keeps its own reference
maximum), so they differ by two independent such errors: their normwise
difference stays within twice sqrt(2) times the RMS (``check_pair``).
"""
from __future__ import annotations

import math

import numpy as np

U = 2.0 ** -8          # bf16
U_FP16 = 2.0 ** -11


def softmax_stats(q, k_pool, v_pool, block_table, seq_lens, scale, ref, page_size=16):
    """Per (row, query head): S1 [B,Hq,D] = sum_t w_t |v_t - ref|,
    S2 [B,Hq] = sum_t w_t^2 ||v_t - ref||^2, W2 [B,Hq] = sum_t w_t^2, with w
    the float64 softmax weights of the inputs (host arrays; fp8 pools as
    already decoded values)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    S1 = np.zeros((B, Hq, D))
    S2 = np.zeros((B, Hq))
    W2 = np.zeros((B, Hq))
    for b in range(B):
        N = int(seq_lens[b])
        if N == 0:
            continue
        t = np.arange(N)
        pages = np.asarray(block_table)[b, t // page_size].astype(np.int64)
        slots = t % page_size
        for g in range(Hkv):
            K = np.asarray(k_pool[pages, g, slots, :], dtype=np.float64)
            V = np.asarray(v_pool[pages, g, slots, :], dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                s = scale * (K @ q[b, h])
                w = np.exp(s - s.max())
                w /= w.sum()
                dv = V - ref[b, h]
                S1[b, h] = w @ np.abs(dv)
                S2[b, h] = (w * w) @ np.einsum("td,td->t", dv, dv)
                W2[b, h] = w @ w
    return S1, S2, W2


def check(got, got_lse, ref, ref_lse, stats, where="", u=U):
    """Raise AssertionError when a result rounded with unit roundoff u breaks
    either bound; returns (max abs error, worst normwise ratio error /
    statistical bound)."""
    S1, S2, W2 = stats
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    err = got - ref
    elem = 1.02 * u / (1 - u) * S1 + u * (1 + u) * np.abs(ref) + 1e-7
    bad = np.abs(err) > elem
    assert not bad.any(), (f"{where}: elementwise bound broken at {np.argwhere(bad)[:3].tolist()}: "
                           f"err {np.abs(err)[bad][:3]} > {elem[bad][:3]}")
    rms = (u / math.sqrt(3.0)) * np.sqrt(S2 + np.einsum("bhd,bhd->bh", ref, ref))
    norm = np.sqrt(np.einsum("bhd,bhd->bh", err, err))
    lim = 2.0 * rms + 1e-6
    ratio = float(np.max(norm / lim)) if norm.size else 0.0
    assert np.all(norm <= lim), (f"{where}: normwise error {float(np.max(norm)):.3e} above twice "
                                 f"its rounding RMS (worst ratio {ratio:.2f})")
    if got_lse is not None:
        got_lse = np.asarray(got_lse, dtype=np.float64)
        inf = np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(got_lse), inf), f"{where}: lse -inf pattern differs"
        if (~inf).any():
            le = np.abs(got_lse[~inf] - ref_lse[~inf])
            assert np.all(le <= u / (1 - u)), f"{where}: lse error {le.max():.3e} > u/(1-u)"
            lim_l = 6.0 * (u / math.sqrt(3.0)) * np.sqrt(W2[~inf]) + 1e-5 + \
                4e-7 * np.abs(ref_lse[~inf])
            assert np.all(le <= lim_l), (f"{where}: lse error {le.max():.3e} above 6 sigma "
                                         f"of its rounding ({float(np.min(lim_l)):.3e})")
    return float(np.max(np.abs(err))) if err.size else 0.0, ratio


def check_pair(a, b, ref, stats, where="", u=U_FP16):
    """Two results of the same inputs under different schedules: per (row,
    head) ||a - b||_2 <= 2 sqrt(2) (u/sqrt 3) sqrt(S2 + ||ref||^2) + 1e-6.
    Returns the worst ratio."""
    _, S2, _ = stats
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    rms = (u / math.sqrt(3.0)) * np.sqrt(S2 + np.einsum("bhd,bhd->bh", ref, ref))
    lim = 2.0 * math.sqrt(2.0) * rms + 1e-6
    d = a - b
    norm = np.sqrt(np.einsum("bhd,bhd->bh", d, d))
    ratio = float(np.max(norm / lim)) if norm.size else 0.0
    assert np.all(norm <= lim), f"{where}: schedules differ by {float(np.max(norm)):.3e} (ratio {ratio:.2f})"
    return ratio
