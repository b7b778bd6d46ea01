"""Pin the float64 oracle to brute force, closed forms, a library special case,
invariances and hand-derived fixtures (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_attend_pins(pin):
    pin(oracle.attend)


def test_hand_fixture():
    with open(os.path.join(GOLDEN, "two_token_attention.json")) as f:
        fx = json.load(f)
    pins.pin_hand_fixture(oracle.attend, fx)


# --------------------------------------------------------------------------- split + merge

@pytest.mark.parametrize("mode,params", [(oracle.MODE_SPLIT, [1, 2, 3, 4, 7, 16]),
                                         (oracle.MODE_WORKQUEUE, [1, 2, 3, 5, 64])])
def test_split_merge_equals_dense(mode, params):
    """The exact merge of split states reproduces the dense result for any split."""
    rng = np.random.default_rng(21)
    c = pins.rand_case(rng, B=3, Hq=4, Hkv=2, D=8, page_size=4, lens=[0, 1, 97])
    ref_out, ref_lse = oracle.attend(c["q"], c["k_pool"], c["v_pool"], c["block_table"],
                                     c["seq_lens"], c["scale"], page_size=4)
    for p in params:
        tasks, offs = oracle.plan_tasks(c["seq_lens"], 2, 4, mode, p)
        out, lse = oracle.split_merge(c["q"], c["k_pool"], c["v_pool"], c["block_table"],
                                      c["seq_lens"], c["scale"], tasks, offs, page_size=4)
        assert pins._rel(out, ref_out) < 1e-12, p
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse))
        assert np.max(np.abs(lse[fin] - ref_lse[fin])) < 1e-12, p


def test_neutral_injection_is_identity():
    """Neutral states (m=-inf, l=0, o=0) change no bit of the merged result."""
    rng = np.random.default_rng(22)
    c = pins.rand_case(rng, B=2, Hq=4, Hkv=2, D=8, page_size=4, lens=[50, 13])
    tasks, offs = oracle.plan_tasks(c["seq_lens"], 2, 4, oracle.MODE_SPLIT, 4)
    args = (c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"], c["scale"],
            tasks, offs)
    a = oracle.split_merge(*args, page_size=4)
    b = oracle.split_merge(*args, page_size=4, extra_neutral=3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_merge_states_two_halves_closed_form():
    """Merging the states of two halves equals the state of the whole range."""
    rng = np.random.default_rng(23)
    q = rng.standard_normal((3, 5))
    K = rng.standard_normal((11, 5))
    V = rng.standard_normal((11, 5))
    m, l, o = oracle.partial_state(q, K, V, 0.7)
    m1, l1, o1 = oracle.partial_state(q, K[:4], V[:4], 0.7)
    m2, l2, o2 = oracle.partial_state(q, K[4:], V[4:], 0.7)
    for h in range(3):
        out, lse = oracle.merge_states([m1[h], m2[h]], [l1[h], l2[h]], np.stack([o1[h], o2[h]]))
        assert np.allclose(out, o[h] / l[h], rtol=1e-13, atol=0)
        assert abs(lse - (m[h] + math.log(l[h]))) < 1e-13
    out, lse = oracle.merge_states([-np.inf, -np.inf], [0.0, 0.0], np.zeros((2, 5)))
    assert np.all(out == 0) and lse == -np.inf


# --------------------------------------------------------------------------- task list

def _check_coverage(seq_lens, Hkv, P, tasks, offs):
    n = [-(-int(x) // P) for x in seq_lens]
    seen = {}
    for b, g, s, c in tasks:
        p0, p1 = s * c, min((s + 1) * c, n[b])
        assert p0 < p1, "empty task emitted"
        for p in range(p0, p1):
            key = (b, g, p)
            assert key not in seen, "page covered twice"
            seen[key] = 1
    assert len(seen) == Hkv * sum(n), "pages missed"
    S = [int(offs[b + 1] - offs[b]) for b in range(len(seq_lens))]
    assert len(tasks) == Hkv * sum(S)
    assert offs[0] == 0 and all(offs[i] <= offs[i + 1] for i in range(len(seq_lens)))


def test_task_list_golden():
    with open(os.path.join(GOLDEN, "task_lists.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        tasks, offs = oracle.plan_tasks(case["seq_lens"], case["Hkv"], 16, case["mode"],
                                        case["param"])
        assert tasks.tolist() == case["tasks"], case["name"]
        assert offs.tolist() == case["split_offsets"], case["name"]


@pytest.mark.parametrize("seed", range(8))
def test_task_list_vs_walking_enumerator(seed):
    rng = np.random.default_rng(300 + seed)
    B = int(rng.integers(1, 9))
    lens = rng.integers(0, 700, size=B)
    lens[rng.integers(0, B)] = 0
    Hkv = int(rng.integers(1, 5))
    for S in (1, 2, 3, 4, 8, 64):
        tasks, offs = oracle.plan_tasks(lens, Hkv, 16, oracle.MODE_SPLIT, S)
        walk = brute.tasks_by_walking(lens, Hkv, 16, lambda b, n: -(-n // S))
        assert tasks.tolist() == walk
        _check_coverage(lens, Hkv, 16, tasks.tolist(), offs)
        assert max(offs[1:] - offs[:-1]) <= S
    for c in (1, 3, 4, 16, 1000):
        tasks, offs = oracle.plan_tasks(lens, Hkv, 16, oracle.MODE_WORKQUEUE, c)
        walk = brute.tasks_by_walking(lens, Hkv, 16, lambda b, n: c)
        assert tasks.tolist() == walk
        _check_coverage(lens, Hkv, 16, tasks.tolist(), offs)


def test_task_list_errors():
    with pytest.raises(ValueError):
        oracle.plan_tasks([16], 1, 16, 7, 1)
    with pytest.raises(ValueError):
        oracle.plan_tasks([16], 1, 16, oracle.MODE_SPLIT, 0)


# --------------------------------------------------------------------------- fp8 KV values

def test_e4m3_decode_spec_values():
    """Values the OCP 8-bit Floating Point Specification (OFP8) states for
    E4M3: largest normal 448 (S.1111.110), smallest normal 2^-6 (S.0001.000),
    largest subnormal 0.875 * 2^-6 (S.0000.111), smallest subnormal 2^-9
    (S.0000.001), zeros of both signs, NaN at S.1111.111 and no infinity."""
    d = oracle.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6
    assert d(0x07) == 0.875 * 2.0 ** -6
    assert d(0x01) == 2.0 ** -9
    assert d(0x00) == 0.0 and not math.copysign(1.0, d(0x00)) < 0
    assert d(0x80) == 0.0 and math.copysign(1.0, d(0x80)) < 0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0x38) == 1.0 and d(0xC0) == -2.0 and d(0x3C) == 1.5
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert not np.isinf(vals).any()
    assert np.isnan(vals).sum() == 2


def test_e4m3_decode_matches_torch():
    """Library special case: torch's float8_e4m3fn holds the same format."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_decode_monotone_and_symmetric():
    """Positive codes 0x00..0x7E increase strictly; the sign bit negates."""
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = oracle.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg[1:], -pos[1:])


def test_attend_k_scale_is_a_softmax_scale():
    """Scaling K by c is scaling the scores by c: attend(k_scale=c) equals
    attend with softmax scale * c (an invariance, to float64 rounding)."""
    rng = np.random.default_rng(5)
    c = pins.rand_case(rng, B=2, Hq=4, Hkv=2, D=8, page_size=4, lens=[7, 30])
    args = (c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"])
    for ks in (0.25, 3.0):
        o1, l1 = oracle.attend(*args, c["scale"], page_size=4, k_scale=ks)
        o2, l2 = oracle.attend(*args, c["scale"] * ks, page_size=4)
        assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_attend_v_scale_scales_the_output_only():
    """out is linear in V and lse does not depend on V."""
    rng = np.random.default_rng(6)
    c = pins.rand_case(rng, B=2, Hq=4, Hkv=1, D=8, page_size=4, lens=[0, 13])
    args = (c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens"], c["scale"])
    o1, l1 = oracle.attend(*args, page_size=4)
    o2, l2 = oracle.attend(*args, page_size=4, v_scale=2.5)
    assert np.max(np.abs(o2 - 2.5 * o1)) < 1e-12
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2))
    fin = ~np.isneginf(l1)
    assert np.max(np.abs(l1[fin] - l2[fin])) < 1e-15


def test_attend_on_codes_is_attend_on_their_values():
    """A uint8 pool is read as E4M3 codes: the result equals attention over
    the codes' values times the scales."""
    rng = np.random.default_rng(7)
    c = pins.rand_case(rng, B=2, Hq=4, Hkv=2, D=8, page_size=4, lens=[5, 18])
    codes_k = rng.integers(0, 256, size=c["k_pool"].shape).astype(np.uint8)
    codes_v = rng.integers(0, 256, size=c["v_pool"].shape).astype(np.uint8)
    # keep the referenced tokens finite: NaN codes only where the rows never read
    nan_k = (codes_k & 0x7F) == 0x7F
    nan_v = (codes_v & 0x7F) == 0x7F
    codes_k[nan_k] = 0x38
    codes_v[nan_v] = 0x38
    vals_k = oracle.e4m3_decode(codes_k)
    vals_v = oracle.e4m3_decode(codes_v)
    args = (c["block_table"], c["seq_lens"], c["scale"])
    o1, l1 = oracle.attend(c["q"], codes_k, codes_v, *args, page_size=4, k_scale=0.5,
                           v_scale=2.0)
    o2, l2 = oracle.attend(c["q"], vals_k * 0.5, vals_v * 2.0, *args, page_size=4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
