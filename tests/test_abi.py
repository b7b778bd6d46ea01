"""C-ABI library on the CPU: it loads, exports every declared symbol, and its
host planner / policy match the oracle bit for bit.  No device calls."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from tests import policy_model_check as pmc
import paged_gqa_decode_pkv_amd as pkv
from workloads import CONFIGS, CALIBRATION_SEED, HELD_OUT_SEEDS, make_lengths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pkv.LIB_PATH)
    declared = _declared_symbols()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(pkv.ABI_SYMBOLS) == declared


def test_version_and_status_strings():
    assert pkv.pkv_abi_version() == pkv.PKV_ABI_VERSION
    hdr = open(os.path.join(ROOT, "include", "pkv.h")).read()
    assert re.search(r"#define PKV_ABI_VERSION (\d+)", hdr).group(1) == str(pkv.PKV_ABI_VERSION)
    for code in range(6):
        assert pkv.pkv_status_string(code)
    assert pkv.pkv_status_string(99) == "unknown status"


def test_page_load_mode_rule():
    """The cache policy of the page loads, a host-side choice per plan: the
    default for 2-byte pools at d = 256, non-temporal K and V for 2-byte plans
    of more than two tasks per CU, non-temporal V otherwise (also for a
    self-planned step, num_tasks < 0)."""
    F16, BF16, F8, BF8 = (pkv.PKV_DTYPE_F16, pkv.PKV_DTYPE_BF16, pkv.PKV_DTYPE_F16_KV_FP8,
                          pkv.PKV_DTYPE_BF16_KV_FP8)
    cases = [
        ((128, F16, 1, 256), 1), ((128, F16, 256, 256), 1), ((128, F16, 512, 256), 1),
        ((128, F16, 513, 256), 2), ((128, BF16, 4752, 256), 2), ((64, F16, 2472, 256), 2),
        ((128, F8, 4752, 256), 1), ((64, BF8, 100000, 256), 1), ((256, F8, 4752, 256), 1),
        ((256, F16, 4752, 256), 0), ((256, BF16, 10, 256), 0),
        ((128, F16, -1, 256), 1), ((256, BF16, -1, 256), 0), ((128, F16, 513, 304), 1),
    ]
    for args, want in cases:
        assert pkv.pkv_page_load_mode(*args) == want, args
    for args, status in [((96, F16, 10, 256), pkv.PKV_ERR_UNSUPPORTED),
                         ((128, 7, 10, 256), pkv.PKV_ERR_INVALID_ARG),
                         ((128, F16, 10, 0), pkv.PKV_ERR_INVALID_ARG)]:
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_page_load_mode(*args)
        assert e.value.status == status


def test_constants_agree_with_oracle():
    assert pkv.PKV_MODE_SPLIT == oracle.MODE_SPLIT
    assert pkv.PKV_MODE_WORKQUEUE == oracle.MODE_WORKQUEUE


# --------------------------------------------------------------------------- plan

def _plan_both(lens, Hkv, maxp, mode, param):
    tasks, offs, slots = pkv.pkv_plan(lens, Hkv, maxp, mode, param)
    rt, ro = oracle.plan_tasks(lens, Hkv, 16, mode, param)
    return tasks, offs, slots, rt, ro


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_plan_bit_exact_on_configs(name):
    cfg = CONFIGS[name]
    for seed in (CALIBRATION_SEED,) + HELD_OUT_SEEDS:
        lens = make_lengths(cfg, seed)
        for mode, params in ((pkv.PKV_MODE_SPLIT, (1, 4, 8, 16, 32, 64, 256)),
                             (pkv.PKV_MODE_WORKQUEUE, (1, 4, 16, 64, 256))):
            for p in params:
                t, o, s, rt, ro = _plan_both(lens, cfg.Hkv, cfg.max_pages_per_row, mode, p)
                assert np.array_equal(t, rt), (name, seed, mode, p)
                assert np.array_equal(o, ro)
                assert s == ro[-1]


@pytest.mark.parametrize("seed", range(20))
def test_plan_bit_exact_random(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 70))
    lens = rng.integers(0, 3000, size=B)
    lens[rng.random(B) < 0.2] = 0
    Hkv = int(rng.choice([1, 2, 4, 8]))
    maxp = int(-(-lens.max() // 16)) + int(rng.integers(0, 3))
    for mode in (pkv.PKV_MODE_SPLIT, pkv.PKV_MODE_WORKQUEUE):
        p = int(rng.integers(1, 300))
        t, o, s, rt, ro = _plan_both(lens, Hkv, maxp, mode, p)
        assert np.array_equal(t, rt) and np.array_equal(o, ro) and s == ro[-1]


def test_plan_empty_and_zero_rows():
    t, o, s = pkv.pkv_plan([0, 0, 0], 8, 4, pkv.PKV_MODE_SPLIT, 4)
    assert t.shape == (0, 4) and o.tolist() == [0, 0, 0, 0] and s == 0
    t, o, s = pkv.pkv_plan([], 8, 4, pkv.PKV_MODE_SPLIT, 4)
    assert t.shape == (0, 4) and o.tolist() == [0]


def test_plan_errors():
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([100], 1, 2, pkv.PKV_MODE_SPLIT, 1)          # 7 pages > 2
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([-1], 1, 2, pkv.PKV_MODE_SPLIT, 1)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([16], 1, 2, 5, 1)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([16], 1, 2, pkv.PKV_MODE_SPLIT, 0)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([16], 1, 2, pkv.PKV_MODE_SPLIT, 1, page_size=32)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    bt = np.array([[3, -1], [0, 9]], dtype=np.int32)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([16, 32], 1, 2, pkv.PKV_MODE_SPLIT, 1, block_table=bt, num_pages=8)
    assert e.value.status == pkv.PKV_ERR_BAD_INDEX          # 9 >= 8
    # entries past n_b are never checked
    t, o, s = pkv.pkv_plan([16, 17], 1, 2, pkv.PKV_MODE_SPLIT, 1,
                           block_table=np.array([[3, -1], [0, 7]], np.int32), num_pages=8)
    assert t.shape[0] == 2


def test_plan_buffer_too_small():
    lib = pkv._load()
    lens = np.array([64, 64], dtype=np.int32)
    tasks = np.zeros((1, 4), dtype=np.int32)
    offs = np.zeros(3, dtype=np.int32)
    nt, ns = ctypes.c_int64(), ctypes.c_int64()
    st = lib.pkv_plan(lens.ctypes.data_as(ctypes.c_void_p), 2, 1, 16, 4, None, 0, 0, 2,
                      tasks.ctypes.data_as(ctypes.c_void_p), 1,
                      offs.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nt), ctypes.byref(ns))
    assert st == pkv.PKV_ERR_BUFFER_TOO_SMALL and nt.value == 4 and ns.value == 4


# --------------------------------------------------------------------------- policy

def _policy_cases():
    rng = np.random.default_rng(5)
    cases = [[32768], [0], [], [100, 0], [16] * 8, [1] * 300, [65536, 1]]
    for name in CONFIGS:
        for seed in (CALIBRATION_SEED,) + HELD_OUT_SEEDS:
            cases.append(make_lengths(CONFIGS[name], seed).tolist())
    for _ in range(60):
        hi = int(rng.choice([300, 5000, 40000, 70000]))
        cases.append(rng.integers(0, hi, size=int(rng.integers(1, 65))).tolist())
    return cases


def test_policy_matches_second_implementation():
    """The library's cost-model policy takes the decision of the independent
    transcription in tests/policy_model_check.py (a cross-implementation
    check, not the oracle), bit for bit, over the workload configs, their
    seeds and random batches."""
    for lens in _policy_cases():
        for cus in (1, 80, 256, 304):
            for Hkv in (1, 8):
                for D in (64, 128):
                    got = pkv.pkv_policy(lens, Hkv, cus, head_dim=D)
                    want = pmc.policy(lens, Hkv, 16, cus, head_dim=D)
                    assert got == tuple(int(x) for x in want), (lens[:4], cus, Hkv, D)


def test_policy_predict_matches_second_implementation_bit_for_bit():
    """The model times themselves agree exactly (same float64 operations, no
    contraction), for every candidate and both launch forms."""
    rng = np.random.default_rng(6)
    for lens in _policy_cases()[::3]:
        for cus in (80, 256):
            for mode, param in [(0, 1), (0, 8), (0, 256), (1, 4), (1, 64), (1, 256),
                                (0, int(rng.integers(1, 500))), (1, int(rng.integers(1, 500)))]:
                for two in (-1, 0, 1):
                    got = pkv.pkv_policy_predict(lens, 8, cus, mode, param, two)
                    shape = pmc.plan_shape(lens, 8, 16, mode, param)
                    t2 = pmc.two_launch(shape, pmc.POLICY_DEFAULTS) if two < 0 else bool(two)
                    want = pmc.predict_us(shape, cus, 128, 16, t2, pmc.POLICY_DEFAULTS)
                    assert got == want, (lens[:4], cus, mode, param, two, got, want)


def test_policy_defaults_are_the_committed_fit():
    """pkv_policy_defaults and the second implementation's defaults hold the
    constants that policy_fit.py fitted on the calibration seed."""
    import json
    fit = json.load(open(os.path.join(ROOT, "paged_gqa_decode_pkv_amd", "calibration",
                                      "mi355x_fit.json")))
    d = pkv.pkv_policy_defaults()
    for name, v in fit["params"].items():
        assert getattr(d, name) == v, name
        assert pmc.POLICY_DEFAULTS[name] == v, name
    assert (d.split_max, d.chunk_min, d.chunk_max, d.fuse_max_splits,
            d.fuse_max_group_splits) == (256, 4, 256, 16, 256)
    for k in ("split_max", "chunk_min", "chunk_max", "fuse_max_splits", "fuse_max_group_splits"):
        assert pmc.POLICY_DEFAULTS[k] == getattr(d, k)


def test_policy_params_and_errors():
    d = pkv.pkv_policy_defaults()
    d.split_max = 8
    d.chunk_max = 2          # below chunk_min: invalid
    with pytest.raises(pkv.PkvError):
        pkv.pkv_policy([32768], 8, 256, params=d)
    d = pkv.pkv_policy_defaults()
    d.chunk_min, d.chunk_max = 1024, 1024
    d.split_max = 8
    # one long row: split, S <= 8; two rows: workqueue, c = 1024 only
    m, p = pkv.pkv_policy([32768], 8, 256, params=d)
    assert m == pkv.PKV_MODE_SPLIT and p in (1, 2, 4, 8)
    assert (m, p) == pmc.policy([32768], 8, 16, 256, split_max=8, chunk_min=1024,
                                chunk_max=1024)
    assert pkv.pkv_policy([32768, 5], 8, 256, params=d) == (pkv.PKV_MODE_WORKQUEUE, 1024)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_policy([-5], 8, 256)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_policy([5], 8, 0)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_policy([5], 8, 256, head_dim=0)
    for field, bad in (("cu_gbps", 0.0), ("hbm_gbps", -1.0), ("alpha", -0.5), ("t0_us", -1.0),
                       ("split_max", 0), ("fuse_max_splits", -1),
                       ("fuse_max_group_splits", -1)):
        d = pkv.pkv_policy_defaults()
        setattr(d, field, bad)
        with pytest.raises(pkv.PkvError):
            pkv.pkv_policy([5000], 8, 256, params=d)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_policy_predict([5000], 8, 256, 7, 4)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_policy_predict([5000], 8, 256, 1, 0)


def test_policy_fit_features_match_the_planner():
    """The calibration tool's closed-form plan features equal the planner's."""
    from paged_gqa_decode_pkv_amd import policy_fit
    rng = np.random.default_rng(8)
    for _ in range(30):
        lens = rng.integers(0, 20000, size=int(rng.integers(1, 20)))
        for mode, param in [(0, 1), (0, 7), (0, 64), (1, 4), (1, 33), (1, 256)]:
            T, P, pmax, maxS = policy_fit.plan_features(lens, 8, mode, param)
            tasks, offs, _ = pkv.pkv_plan(lens, 8, 2048, mode, param)
            n = -(-lens // 16)
            pages = [min((s + 1) * c, n[b]) - s * c for b, g, s, c in tasks]
            assert T == len(tasks) and P == sum(pages) and pmax == max(pages, default=0)
            assert maxS == (int(np.max(np.diff(offs))) if len(offs) > 1 else 0)


# --------------------------------------------------------------------------- workspace, decode arg checks

def test_workspace_size():
    hdr = pkv.WORKSPACE_HEADER_BYTES
    assert pkv.pkv_workspace_size(0, 32, 128) == hdr
    n = pkv.pkv_workspace_size(10, 32, 128)
    assert n >= hdr + 10 * 32 * 130 * 4 and n % 256 == 0
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    assert re.search(r"#define PKV_WORKSPACE_HEADER_BYTES %d\b" % hdr, text)


def test_decode_rejects_bad_scalars_before_touching_the_device():
    lib = pkv._load()
    common = dict(q=None, k=None, v=None)
    def call(B=1, Hq=4, Hkv=1, D=64, P=16, scale=0.125, dtype=pkv.PKV_DTYPE_F16, ks=1.0, vs=1.0):
        return lib.pkv_decode(None, None, None, 0, None, 1, None, None, 0, None, 0, B, Hq, Hkv, D,
                              P, dtype, scale, ks, vs, None, None, None, 0, None)
    assert call(D=96) == pkv.PKV_ERR_UNSUPPORTED
    assert call(D=256, Hq=16, Hkv=1) == pkv.PKV_ERR_INVALID_ARG   # G = 16 at d = 256; null pointers
    assert call(D=256, Hq=4, Hkv=1) == pkv.PKV_ERR_INVALID_ARG    # supported; null pointers
    assert call(Hq=32, Hkv=1) == pkv.PKV_ERR_UNSUPPORTED     # G = 32
    assert call(P=32) == pkv.PKV_ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=4) == pkv.PKV_ERR_UNSUPPORTED      # Hq % Hkv
    assert call(Hq=48, Hkv=3) == pkv.PKV_ERR_INVALID_ARG     # G = 16, supported; null pointers
    assert call(Hq=36, Hkv=3) == pkv.PKV_ERR_UNSUPPORTED     # G = 12
    assert call(dtype=4) == pkv.PKV_ERR_UNSUPPORTED          # no such element type
    assert call(dtype=-1) == pkv.PKV_ERR_UNSUPPORTED
    for dt in (pkv.PKV_DTYPE_BF16, pkv.PKV_DTYPE_F16_KV_FP8, pkv.PKV_DTYPE_BF16_KV_FP8):
        assert call(dtype=dt) == pkv.PKV_ERR_INVALID_ARG     # supported, null pointers
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("nan"), 1.0), (1.0, float("inf"))):
        assert call(ks=ks, vs=vs) == pkv.PKV_ERR_INVALID_ARG   # scales finite and > 0
    assert call(B=-1) == pkv.PKV_ERR_INVALID_ARG
    assert call(scale=float("nan")) == pkv.PKV_ERR_INVALID_ARG
    assert call(B=0) == pkv.PKV_OK                           # nothing to do
    assert call(B=1) == pkv.PKV_ERR_INVALID_ARG              # null pointers
    del common


def test_device_plan_workspace_size_and_host_checks():
    """pkv_decode_device_plan's capacity checks run on the host, before any
    device call (so they work here without a GPU)."""
    hdr_bytes, B, Hq, Hkv, D, cap = 64, 8, 32, 8, 128, 16
    n = pkv.pkv_workspace_size_device_plan(B, Hq, Hkv, D, cap)
    base = pkv.pkv_workspace_size(B * cap, Hq, D)
    assert n % 256 == 0
    assert n >= base + hdr_bytes + ((B + 1) * 4 + 15) // 16 * 16 + Hkv * B * cap * 16
    with pytest.raises(pkv.PkvError):
        pkv.pkv_workspace_size_device_plan(B, Hq, Hkv, D, 0)
    lib = pkv._load()

    def call(mode, param, max_splits, B=2, maxp=1024):
        return lib.pkv_decode_device_plan(None, None, None, 0, None, maxp, None, B, 32, 8, 128, 16,
                                          pkv.PKV_DTYPE_F16, 0.1, 1.0, 1.0, mode, param,
                                          max_splits, None, 256, None, None, None, 0, None)
    assert call(-1, 0, 8, B=0) == pkv.PKV_OK                   # nothing to do
    assert call(2, 1, 8) == pkv.PKV_ERR_INVALID_ARG            # unknown mode
    assert call(-1, 0, 0) == pkv.PKV_ERR_INVALID_ARG           # no capacity
    assert call(0, 16, 8) == pkv.PKV_ERR_INVALID_ARG           # S = 16 > 8 splits
    assert call(1, 4, 8) == pkv.PKV_ERR_INVALID_ARG            # 1024 / 4 = 256 splits > 8
    assert call(1, 128, 8) == pkv.PKV_ERR_INVALID_ARG          # fits, but null pointers
    assert call(-1, 0, 8) == pkv.PKV_ERR_INVALID_ARG           # null pointers


def test_step_args_layout_matches_c(tmp_path):
    """The ctypes mirror of pkv_step_args has the C field offsets and size."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in pkv.pkv_step_args._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "pkv.h"', 'int main(void) {',
           '  printf("%zu\\n", sizeof(pkv_step_args));']
    src += [f'  printf("%zu\\n", offsetof(pkv_step_args, {f}));' for f in fields]
    src += ['  return 0;', '}']
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(pkv.pkv_step_args)
    for f, off in zip(fields, got[1:]):
        assert getattr(pkv.pkv_step_args, f).offset == off, f


def test_runner_rejects_bad_args_without_device():
    lib = pkv._load()
    h = ctypes.c_void_p()
    assert lib.pkv_runner_create(0, None, 0, ctypes.byref(h)) == pkv.PKV_ERR_INVALID_ARG
    assert lib.pkv_runner_step(None, None) == pkv.PKV_ERR_INVALID_ARG
    assert lib.pkv_runner_destroy(None) == pkv.PKV_OK


def test_library_allocates_no_device_memory():
    """The built library imports no device allocator: every device buffer
    (the workspace and the runner's copy of the plan included) belongs to the
    caller.  (Pinned host memory for the runner's plan ring is allowed.)"""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", pkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    for sym in ("hipMalloc", "hipMallocAsync", "hipMallocManaged", "hipExtMallocWithFlags",
                "hipMallocPitch", "hipMalloc3D", "hipFree", "hipFreeAsync"):
        assert sym not in imported, sym
    assert "hipHostMalloc" in imported
