"""Checks that pin the float64 oracle to something other than itself.

Each ``pin_*`` takes an ``attend(q, k_pool, v_pool, block_table, seq_lens,
scale, page_size)`` implementation and raises AssertionError if it disagrees
with brute force, a closed form, a library special case or an invariance.
``tests/test_oracle_pins.py`` runs them on the oracle; ``tests/
test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires at least one pin to fail for every mutant.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import brute


def rand_case(rng, B=2, Hq=4, Hkv=2, D=8, page_size=4, max_n=40, pool_extra=3,
              lens=None, dtype=np.float64, poison=True):
    """Small random paged batch (numpy).  Unreferenced pages / tail slots hold NaN."""
    if lens is None:
        lens = rng.integers(1, max_n + 1, size=B)
    lens = np.asarray(lens, dtype=np.int64)
    n = -(-lens // page_size)
    maxp = max(int(n.max(initial=0)), 1)
    pool = int(n.sum()) + pool_extra
    perm = rng.permutation(pool)
    bt = np.full((B, maxp), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        bt[b, :n[b]] = perm[off:off + n[b]]
        off += n[b]
    fillv = np.nan if poison else 0.0
    k = np.full((pool, Hkv, page_size, D), fillv)
    v = np.full((pool, Hkv, page_size, D), fillv)
    used = perm[:off]
    k[used] = rng.standard_normal((off, Hkv, page_size, D))
    v[used] = rng.standard_normal((off, Hkv, page_size, D))
    for b in range(B):
        r = lens[b] % page_size
        if lens[b] and r:
            last = bt[b, (lens[b] - 1) // page_size]
            k[last, :, r:] = fillv
            v[last, :, r:] = fillv
    q = rng.standard_normal((B, Hq, D))
    return dict(q=q.astype(dtype), k_pool=k.astype(dtype), v_pool=v.astype(dtype),
                block_table=bt, seq_lens=lens, scale=1.0 / math.sqrt(D), page_size=page_size)


def _call(attend, c, **over):
    a = dict(c)
    a.update(over)
    return attend(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["seq_lens"],
                  a["scale"], page_size=a["page_size"])


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------

def pin_brute_force(attend, seeds=range(6)):
    """Pure-Python loops (math.fsum, math.exp) on tiny ragged shapes."""
    shapes = [(1, 1, 1, 3, 4), (2, 4, 2, 8, 4), (2, 4, 1, 5, 16), (1, 8, 2, 4, 4),
              (2, 2, 2, 6, 16), (1, 4, 4, 3, 4)]
    for seed, (B, Hq, Hkv, D, P) in zip(seeds, shapes):
        rng = np.random.default_rng(1000 + seed)
        c = rand_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, page_size=P, max_n=40)
        out, lse = _call(attend, c)
        bo, bl = brute.attend_loops(c["q"].tolist(), c["k_pool"].tolist(), c["v_pool"].tolist(),
                                    c["block_table"].tolist(), c["seq_lens"].tolist(),
                                    c["scale"], c["page_size"])
        assert _rel(out, bo) < 1e-12, ("brute out", seed)
        assert _rel(lse, bl) < 1e-12, ("brute lse", seed)


def pin_constant_v(attend):
    """V_t = c_g for every token of KV head g  =>  out[b,h] = c_{floor(h/G)} exactly."""
    rng = np.random.default_rng(7)
    c = rand_case(rng, B=2, Hq=6, Hkv=3, D=5, page_size=4, max_n=30)
    cvec = rng.standard_normal((3, 5))
    v = np.array(c["v_pool"])
    for g in range(3):
        v[:, g, :, :] = np.where(np.isnan(v[:, g, :, :]), np.nan, cvec[g])
    out, _ = _call(attend, c, v_pool=v)
    for h in range(6):
        assert np.allclose(out[:, h], cvec[h // 2], rtol=0, atol=1e-14), ("const V", h)


def pin_single_token(attend):
    """N = 1  =>  out = v_0 and lse = scale * <q, k_0>."""
    rng = np.random.default_rng(8)
    c = rand_case(rng, B=2, Hq=4, Hkv=2, D=6, page_size=4, lens=[1, 1])
    out, lse = _call(attend, c)
    for b in range(2):
        page = c["block_table"][b, 0]
        for h in range(4):
            g = h // 2
            assert np.array_equal(out[b, h], c["v_pool"][page, g, 0]), ("N=1 out", b, h)
            ref = c["scale"] * math.fsum(c["q"][b, h] * c["k_pool"][page, g, 0])
            assert abs(lse[b, h] - ref) <= 1e-14 * max(1.0, abs(ref)), ("N=1 lse", b, h)


def pin_zero_query(attend):
    """q = 0  =>  out = mean_t V_t and lse = log N exactly (uniform weights)."""
    rng = np.random.default_rng(9)
    lens = [37, 16, 5]
    c = rand_case(rng, B=3, Hq=2, Hkv=1, D=4, page_size=16, lens=lens)
    q0 = np.zeros_like(c["q"])
    out, lse = _call(attend, c, q=q0)
    for b, N in enumerate(lens):
        toks = [c["v_pool"][c["block_table"][b, t // 16], 0, t % 16] for t in range(N)]
        mean = np.array([math.fsum(x[j] for x in toks) / N for j in range(4)])
        for h in range(2):
            assert _rel(out[b, h], mean) < 1e-13, ("q=0 mean", b)
            assert lse[b, h] == math.log(N), ("q=0 lse", b)


def pin_head_map(attend):
    """V = g+1 on KV head g  =>  out[h] = floor(h/G)+1 (contiguous groups)."""
    rng = np.random.default_rng(10)
    Hq, Hkv = 8, 2
    c = rand_case(rng, B=1, Hq=Hq, Hkv=Hkv, D=3, page_size=4, max_n=20)
    v = np.array(c["v_pool"])
    for g in range(Hkv):
        v[:, g] = np.where(np.isnan(v[:, g]), np.nan, float(g + 1))
    out, _ = _call(attend, c, v_pool=v)
    G = Hq // Hkv
    for h in range(Hq):
        assert np.allclose(out[0, h], h // G + 1, rtol=1e-14, atol=0), ("head map", h)


def pin_page_indicator(attend):
    """Physical page holding logical page j of the row stores V = e_j; q = 0.

    Then out[j] = (#tokens of the row in logical page j) / N.  Unreferenced
    pages and tail slots store e_{D-1} (a column no logical page uses), so any
    token read past N_b or through a wrong page shows up in out[D-1].
    """
    P, D = 4, 8
    lens = [13, 4, 1, 25]
    rng = np.random.default_rng(11)
    c = rand_case(rng, B=4, Hq=2, Hkv=1, D=D, page_size=P, lens=lens, poison=False)
    pool = c["k_pool"].shape[0]
    v = np.zeros((pool, 1, P, D))
    v[:, :, :, D - 1] = 1.0
    for b, N in enumerate(lens):
        n = -(-N // P)
        for j in range(n):
            page = c["block_table"][b, j]
            v[page] = 0.0
            for slot in range(P):
                t = j * P + slot
                v[page, 0, slot, j if t < N else D - 1] = 1.0
    out, _ = _call(attend, c, q=np.zeros_like(c["q"]), v_pool=v)
    for b, N in enumerate(lens):
        n = -(-N // P)
        want = np.zeros(D)
        for j in range(n):
            want[j] = (min(N, (j + 1) * P) - j * P) / N
        for h in range(2):
            assert np.allclose(out[b, h], want, rtol=0, atol=1e-15), ("page indicator", b)


def pin_library_sdpa(attend):
    """Identity block table = dense layout: equals torch SDPA (float64, CPU) with
    KV heads repeated per group, and lse equals torch.logsumexp of the scores."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, P, N = 2, 8, 2, 16, 16, 80
    n = N // P
    k = rng.standard_normal((B * n, Hkv, P, D))
    v = rng.standard_normal((B * n, Hkv, P, D))
    q = rng.standard_normal((B, Hq, D))
    bt = np.arange(B * n).reshape(B, n)
    scale = 1.0 / math.sqrt(D)
    out, lse = attend(q, k, v, bt, np.array([N, N]), scale, page_size=P)
    # dense [B, Hkv, N, D]
    kd = torch.from_numpy(k.reshape(B, n, Hkv, P, D).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, N, D))
    vd = torch.from_numpy(v.reshape(B, n, Hkv, P, D).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, N, D))
    G = Hq // Hkv
    kr = kd.repeat_interleave(G, dim=1).contiguous()
    vr = vd.repeat_interleave(G, dim=1).contiguous()
    qt = torch.from_numpy(q).unsqueeze(2)                        # [B, Hq, 1, D]
    ref = F.scaled_dot_product_attention(qt, kr, vr, scale=scale).squeeze(2).numpy()
    assert _rel(out, ref) < 1e-12, "sdpa out"
    scores = torch.matmul(qt, kr.transpose(-1, -2).contiguous()).squeeze(2) * scale
    ref_lse = torch.logsumexp(scores, dim=-1).numpy()
    assert _rel(lse, ref_lse) < 1e-13, "logsumexp"


def pin_permutation(attend):
    """Relabelling pool pages (and the block table with them) changes nothing."""
    from workloads import relabel_pages

    rng = np.random.default_rng(13)
    c = rand_case(rng, B=2, Hq=4, Hkv=2, D=8, page_size=4, max_n=40, pool_extra=9)
    out, lse = _call(attend, c)
    c2 = relabel_pages(c, np.random.default_rng(14))
    out2, lse2 = _call(attend, c2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "relabel"


def pin_empty_row(attend):
    """N_b = 0  =>  out = 0, lse = -inf; other rows unaffected."""
    rng = np.random.default_rng(15)
    c = rand_case(rng, B=3, Hq=2, Hkv=1, D=4, page_size=4, lens=[0, 9, 0])
    out, lse = _call(attend, c)
    for b in (0, 2):
        assert np.all(out[b] == 0.0) and np.all(np.isneginf(lse[b])), "empty row"
    assert np.all(np.isfinite(out[1])), "non-empty row"


def pin_hand_fixture(attend, fixture):
    """Hand-derived two-token example stored under tests/golden/."""
    f = fixture
    q = np.array(f["q"], dtype=np.float64)
    k = np.array(f["k_pool"], dtype=np.float64)
    v = np.array(f["v_pool"], dtype=np.float64)
    out, lse = attend(q, k, v, np.array(f["block_table"]), np.array(f["seq_lens"]),
                      f["scale"], page_size=f["page_size"])
    assert np.allclose(out, np.array(f["out"]), rtol=0, atol=1e-14), "fixture out"
    assert np.allclose(lse, np.array(f["lse"]), rtol=0, atol=1e-14), "fixture lse"


ALL_PINS = [pin_brute_force, pin_constant_v, pin_single_token, pin_zero_query, pin_head_map,
            pin_page_indicator, pin_library_sdpa, pin_permutation, pin_empty_row]
