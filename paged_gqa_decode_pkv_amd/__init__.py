"""Python binding of libpkv.so: paged GQA decode attention on MI355X (gfx950).

Argument marshalling only.  Every step of the decode path runs in the
library: the host planner and policy (C++) and the HIP kernels.  PyTorch
supplies device memory and streams.  The functions mirror the C ABI of
``include/pkv.h`` under the same names.

If ``libpkv.so`` has not been built (``python -m paged_gqa_decode_pkv_amd.build``),
the first call raises ``ImportError``.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB_PATH selects another build of the same library (the host-side
# sanitizer build of paged_gqa_decode_pkv_amd/sanitize.py).
LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(_HERE, "libpkv.so")

PKV_ABI_VERSION = 6               # include/pkv.h; the argument lists below follow it
PKV_OK = 0
PKV_ERR_INVALID_ARG = 1
PKV_ERR_UNSUPPORTED = 2
PKV_ERR_BUFFER_TOO_SMALL = 3
PKV_ERR_BAD_INDEX = 4
PKV_ERR_HIP = 5
PKV_ERR_SCRATCH_TOO_SMALL = 6
PKV_STATIC_SCRATCH_BYTES = 16 << 20   # PKV_STATIC_SCRATCH_BYTES

PKV_DTYPE_F16 = 0
PKV_DTYPE_BF16 = 1
PKV_DTYPE_F16_KV_FP8 = 2       # q / out fp16, K / V pools fp8 E4M3 (torch.float8_e4m3fn)
PKV_DTYPE_BF16_KV_FP8 = 3      # q / out bf16, K / V pools fp8 E4M3
PKV_MODE_SPLIT = 0
PKV_MODE_WORKQUEUE = 1

PKV_DEVERR_TASK = 1
PKV_DEVERR_PAGE = 2
PKV_DEVERR_ROW = 4
PKV_DEVERR_SLOT = 8

PAGE_SIZE = 16
WORKSPACE_HEADER_BYTES = 65536      # PKV_WORKSPACE_HEADER_BYTES
PKV_MAX_FUSED_GROUPS = (WORKSPACE_HEADER_BYTES - 256) // 4   # PKV_MAX_FUSED_GROUPS

# Every symbol include/pkv.h declares.
ABI_SYMBOLS = (
    "pkv_abi_version", "pkv_status_string", "pkv_last_hip_error", "pkv_page_load_mode",
    "pkv_policy_defaults",
    "pkv_policy", "pkv_policy_predict", "pkv_plan", "pkv_workspace_size", "pkv_workspace_init",
    "pkv_workspace_error_flags", "pkv_decode", "pkv_decode_static", "pkv_decode_splits",
    "pkv_merge",
    "pkv_workspace_size_device_plan", "pkv_decode_device_plan", "pkv_device_plan_read",
    "pkv_runner_create", "pkv_runner_step", "pkv_runner_destroy", "pkv_runner_last_plan",
)


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {pkv_status_string(status)} (status {status})"
        if status == PKV_ERR_HIP:
            msg += f", hipError {pkv_last_hip_error()}"
        super().__init__(msg)


class pkv_policy_params(ctypes.Structure):
    """Mirror of pkv_policy_params in include/pkv.h."""
    _fields_ = [("split_max", ctypes.c_int32), ("chunk_min", ctypes.c_int32),
                ("chunk_max", ctypes.c_int32), ("fuse_max_splits", ctypes.c_int32),
                ("fuse_max_group_splits", ctypes.c_int32),
                ("t0_us", ctypes.c_double), ("t_round_us", ctypes.c_double),
                ("alpha", ctypes.c_double), ("cu_gbps", ctypes.c_double),
                ("hbm_gbps", ctypes.c_double), ("t_two_us", ctypes.c_double),
                ("t_two_split_us", ctypes.c_double), ("t_fused_split_us", ctypes.c_double)]

    MODEL = ("t0_us", "t_round_us", "alpha", "cu_gbps", "hbm_gbps", "t_two_us",
             "t_two_split_us", "t_fused_split_us")


class pkv_step_args(ctypes.Structure):
    """Mirror of pkv_step_args in include/pkv.h (same field order and types)."""
    _fields_ = [
        ("seq_lens_host", ctypes.c_void_p), ("B", ctypes.c_int32), ("mode", ctypes.c_int32),
        ("param", ctypes.c_int32), ("two_launch", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64), ("block_table", ctypes.c_void_p),
        ("max_pages_per_row", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
        ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p),
        ("event_before_decode", ctypes.c_void_p), ("event_after_decode", ctypes.c_void_p),
        ("chosen_mode", ctypes.c_int32), ("chosen_param", ctypes.c_int32),
        ("chosen_two_launch", ctypes.c_int32), ("max_splits", ctypes.c_int32),
        ("num_tasks", ctypes.c_int64), ("num_partial_slots", ctypes.c_int64),
        ("workspace_bytes_needed", ctypes.c_size_t),
    ]


_lib = None
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_gqa_decode_pkv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    sig = {
        "pkv_abi_version": ([], ctypes.c_int),
        "pkv_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "pkv_last_hip_error": ([], ctypes.c_int),
        "pkv_page_load_mode": ([i32, i32, i64, i32, _i32p], ctypes.c_int),
        "pkv_policy_defaults": ([ctypes.POINTER(pkv_policy_params)], ctypes.c_int),
        "pkv_policy": ([_vp, i32, i32, i32, i32, i32, ctypes.POINTER(pkv_policy_params), _i32p,
                        _i32p],
                       ctypes.c_int),
        "pkv_policy_predict": ([_vp, i32, i32, i32, i32, i32, ctypes.POINTER(pkv_policy_params),
                                i32, i32, i32, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "pkv_plan": ([_vp, i32, i32, i32, i32, _vp, i64, i32, i32, _vp, i64, _vp, _i64p, _i64p],
                     ctypes.c_int),
        "pkv_workspace_size": ([i64, i32, i32, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "pkv_workspace_init": ([_vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "pkv_workspace_error_flags": ([_vp, ctypes.POINTER(ctypes.c_uint32), _vp], ctypes.c_int),
        "pkv_decode": ([_vp, _vp, _vp, i64, _vp, i32, _vp, _vp, i64, _vp, i64, i32, i32, i32, i32,
                        i32, i32, ctypes.c_float, ctypes.c_float, ctypes.c_float, _vp, _vp, _vp,
                        ctypes.c_size_t, _vp], ctypes.c_int),
        "pkv_merge": ([_vp, i64, i32, i32, i32, i32, i32, _vp, _vp, _vp, ctypes.c_size_t, _vp],
                      ctypes.c_int),
        "pkv_workspace_size_device_plan": ([i32, i32, i32, i32, i32,
                                            ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "pkv_decode_device_plan": ([_vp, _vp, _vp, i64, _vp, i32, _vp, i32, i32, i32, i32, i32,
                                    i32, ctypes.c_float, ctypes.c_float, ctypes.c_float, i32, i32,
                                    i32,
                                    ctypes.POINTER(pkv_policy_params), i32, _vp, _vp, _vp,
                                    ctypes.c_size_t, _vp], ctypes.c_int),
        "pkv_device_plan_read": ([_vp, ctypes.c_size_t, i32, i32, i32, i32, i32, _i32p, _vp, _vp,
                                  i64, _vp], ctypes.c_int),
        "pkv_runner_create": ([i32, ctypes.POINTER(pkv_policy_params), i32, ctypes.POINTER(_vp)],
                              ctypes.c_int),
        "pkv_runner_step": ([_vp, ctypes.POINTER(pkv_step_args)], ctypes.c_int),
        "pkv_runner_destroy": ([_vp], ctypes.c_int),
        "pkv_runner_last_plan": ([_vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64p, _i32p],
                                 ctypes.c_int),
    }
    sig["pkv_decode_splits"] = sig["pkv_decode"]
    sig["pkv_decode_static"] = (sig["pkv_decode"][0][:-3] + [_vp], ctypes.c_int)
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    got = lib.pkv_abi_version()
    if got != PKV_ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {got}, the binding expects "
                          f"{PKV_ABI_VERSION}; rebuild with `python -m paged_gqa_decode_pkv_amd.build`")
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != PKV_OK:
        raise PkvError(status, where)


def _host_i32(x) -> np.ndarray:
    if hasattr(x, "cpu"):
        x = x.cpu().numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------- host calls

def pkv_abi_version() -> int:
    return _load().pkv_abi_version()


def pkv_status_string(status: int) -> str:
    return _load().pkv_status_string(status).decode()


def pkv_last_hip_error() -> int:
    return _load().pkv_last_hip_error()


def pkv_page_load_mode(head_dim: int, dtype: int, num_tasks: int, num_cus: int) -> int:
    """Cache policy of the decode kernel's page loads for a plan: 0 default,
    1 non-temporal V loads, 2 non-temporal K and V loads (num_tasks < 0: a
    self-planned step); see pkv_page_load_mode in include/pkv.h."""
    mode = ctypes.c_int32()
    _check(_load().pkv_page_load_mode(head_dim, dtype, num_tasks, num_cus, ctypes.byref(mode)),
           "pkv_page_load_mode")
    return mode.value


def pkv_policy_defaults() -> pkv_policy_params:
    p = pkv_policy_params()
    _check(_load().pkv_policy_defaults(ctypes.byref(p)), "pkv_policy_defaults")
    return p


def pkv_policy(seq_lens, Hkv: int, num_cus: int, params: Optional[pkv_policy_params] = None,
               page_size: int = PAGE_SIZE, head_dim: int = 128) -> Tuple[int, int]:
    """(mode, param) for this batch; see pkv_policy in include/pkv.h."""
    sl = _host_i32(seq_lens)
    mode, param = ctypes.c_int32(), ctypes.c_int32()
    pp = ctypes.byref(params) if params is not None else None
    _check(_load().pkv_policy(_ptr(sl), sl.size, Hkv, head_dim, page_size, num_cus, pp,
                              ctypes.byref(mode), ctypes.byref(param)), "pkv_policy")
    return mode.value, param.value


def pkv_policy_predict(seq_lens, Hkv: int, num_cus: int, mode: int, param: int,
                       two_launch: int = -1, params: Optional[pkv_policy_params] = None,
                       page_size: int = PAGE_SIZE, head_dim: int = 128) -> float:
    """Model time (us) of one candidate; see pkv_policy_predict in include/pkv.h."""
    sl = _host_i32(seq_lens)
    us = ctypes.c_double()
    pp = ctypes.byref(params) if params is not None else None
    _check(_load().pkv_policy_predict(_ptr(sl), sl.size, Hkv, head_dim, page_size, num_cus, pp,
                                      mode, param, two_launch, ctypes.byref(us)),
           "pkv_policy_predict")
    return us.value


def pkv_plan(seq_lens, Hkv: int, max_pages_per_row: int, mode: int, param: int,
             block_table=None, num_pages: int = 0, page_size: int = PAGE_SIZE,
             tasks_out: Optional[np.ndarray] = None, offsets_out: Optional[np.ndarray] = None):
    """Compact task list.  Returns (tasks int32 [T,4], split_offsets int32 [B+1],
    num_partial_slots).  ``tasks_out`` / ``offsets_out`` (e.g. pinned host
    memory viewed as numpy) are filled in place when given and large enough."""
    lib = _load()
    sl = _host_i32(seq_lens)
    B = sl.size
    bt = _host_i32(block_table) if block_table is not None else None
    if bt is not None and bt.shape != (B, max_pages_per_row):
        raise ValueError("block_table shape must be [B, max_pages_per_row]")
    nt, ns = ctypes.c_int64(), ctypes.c_int64()
    args = (_ptr(sl), B, Hkv, page_size, max_pages_per_row, _ptr(bt) if bt is not None else None,
            num_pages)
    _check(lib.pkv_plan(*args, mode, param, None, 0, None, ctypes.byref(nt), ctypes.byref(ns)),
           "pkv_plan")
    T = nt.value
    if tasks_out is not None and tasks_out.size >= 4 * T and tasks_out.dtype == np.int32:
        tasks = tasks_out.reshape(-1)[:4 * T].reshape(T, 4)
    else:
        tasks = np.empty((T, 4), dtype=np.int32)
    if offsets_out is not None and offsets_out.size >= B + 1 and offsets_out.dtype == np.int32:
        offs = offsets_out.reshape(-1)[:B + 1]
    else:
        offs = np.empty(B + 1, dtype=np.int32)
    _check(lib.pkv_plan(*args, mode, param, _ptr(tasks), T, _ptr(offs), ctypes.byref(nt),
                        ctypes.byref(ns)), "pkv_plan")
    return tasks, offs, ns.value


def pkv_workspace_size(num_partial_slots: int, Hq: int, head_dim: int) -> int:
    n = ctypes.c_size_t()
    _check(_load().pkv_workspace_size(num_partial_slots, Hq, head_dim, ctypes.byref(n)),
           "pkv_workspace_size")
    return n.value


# --------------------------------------------------------------------------- device calls

def current_stream_ptr() -> int:
    """Raw pointer (hipStream_t) of torch's current stream on the current
    device: the value of ``torch.cuda.current_stream().cuda_stream`` without
    building a Stream object, which takes about 3 us of Python per call, as
    much as the rest of a step's enqueue (policy, plan and launch).  Falls
    back to the public call where torch lacks the raw getter."""
    import torch
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is None:
        return torch.cuda.current_stream().cuda_stream
    return get(torch.cuda.current_device())


def _stream_ptr(stream):
    return ctypes.c_void_p(current_stream_ptr() if stream is None else stream.cuda_stream)


def _elem_dtype(*tensors):
    """pkv_dtype code of fp16 / bf16 tensors that must all share one type."""
    import torch
    codes = {torch.float16: PKV_DTYPE_F16, torch.bfloat16: PKV_DTYPE_BF16}
    dt = tensors[0].dtype
    if dt not in codes:
        raise TypeError(f"q, the pools and out must be float16 or bfloat16, got {dt}")
    for t in tensors[1:]:
        if t.dtype != dt:
            raise TypeError(f"q, the pools and out must share one dtype ({dt} vs {t.dtype})")
    return codes[dt], dt


def _fp8_dtype():
    import torch
    return getattr(torch, "float8_e4m3fn", None)


def _dtypes(q, k_pool, v_pool, out):
    """(pkv_dtype code, q / out torch dtype, pool torch dtype).  q and out are
    float16 or bfloat16; the pools are that same type or float8_e4m3fn."""
    import torch
    e = q.dtype
    if e not in (torch.float16, torch.bfloat16):
        raise TypeError(f"q must be float16 or bfloat16, got {e}")
    if out.dtype != e:
        raise TypeError(f"q and out must share one dtype ({e} vs {out.dtype})")
    kv = k_pool.dtype
    if v_pool.dtype != kv:
        raise TypeError(f"k_pool and v_pool must share one dtype ({kv} vs {v_pool.dtype})")
    f16 = e == torch.float16
    if kv == e:
        return (PKV_DTYPE_F16 if f16 else PKV_DTYPE_BF16), e, kv
    if kv == _fp8_dtype():
        return (PKV_DTYPE_F16_KV_FP8 if f16 else PKV_DTYPE_BF16_KV_FP8), e, kv
    raise TypeError(f"the pools must be {e} or float8_e4m3fn, got {kv}")


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def pkv_workspace_init(workspace, stream=None):
    import torch
    _dev(workspace, torch.uint8, "workspace")
    _check(_load().pkv_workspace_init(ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                      _stream_ptr(stream)), "pkv_workspace_init")


def pkv_workspace_error_flags(workspace, stream=None) -> int:
    flags = ctypes.c_uint32()
    _check(_load().pkv_workspace_error_flags(ctypes.c_void_p(workspace.data_ptr()),
                                             ctypes.byref(flags), _stream_ptr(stream)),
           "pkv_workspace_error_flags")
    return flags.value


def _decode_args(q, k_pool, v_pool, block_table, seq_lens, tasks, split_offsets,
                 num_partial_slots, scale, out, workspace, lse, stream, k_scale=1.0, v_scale=1.0):
    """Checked ctypes argument tuple shared by pkv_decode and pkv_decode_splits.

    q [B,Hq,d] fp16, k_pool / v_pool [pages,Hkv,16,d] fp16, block_table
    [B,max_pages] int32, seq_lens [B] int32, tasks [T,4] int32, split_offsets
    [B+1] int32, out [B,Hq,d] fp16, lse [B,Hq] fp32 or None, workspace uint8.
    """
    import torch
    i32 = torch.int32
    code, f16, kvt = _dtypes(q, k_pool, v_pool, out)
    B, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_pool.shape
    if Dk != D or tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != (B, Hq, D):
        raise ValueError("shape mismatch between q, k_pool, v_pool and out")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    if split_offsets.shape != (B + 1,) or tasks.dim() != 2 or tasks.shape[1] != 4:
        raise ValueError("tasks must be [T, 4] and split_offsets [B+1]")
    if lse is not None and tuple(lse.shape) != (B, Hq):
        raise ValueError("lse must be [B, Hq]")
    args = (
        _dev(q, f16, "q"), _dev(k_pool, kvt, "k_pool"), _dev(v_pool, kvt, "v_pool"), num_pages,
        _dev(block_table, i32, "block_table"), block_table.shape[1],
        _dev(seq_lens, i32, "seq_lens"), _dev(tasks, i32, "tasks"), tasks.shape[0],
        _dev(split_offsets, i32, "split_offsets"), num_partial_slots, B, Hq, Hkv, D, P, code,
        float(scale), float(k_scale), float(v_scale), _dev(out, f16, "out"),
        _dev(lse, torch.float32, "lse") if lse is not None else None,
    ) + ((_dev(workspace, torch.uint8, "workspace"), workspace.numel())
         if workspace is not None else ()) + (_stream_ptr(stream),)
    return args


def pkv_decode(q, k_pool, v_pool, block_table, seq_lens, tasks, split_offsets,
               num_partial_slots: int, scale: float, out, workspace, lse=None, stream=None,
               k_scale: float = 1.0, v_scale: float = 1.0):
    """Enqueue decode + merge on ``stream``; see pkv_decode in include/pkv.h."""
    args = _decode_args(q, k_pool, v_pool, block_table, seq_lens, tasks, split_offsets,
                        num_partial_slots, scale, out, workspace, lse, stream, k_scale, v_scale)
    _check(_load().pkv_decode(*args), "pkv_decode")


def pkv_decode_static(q, k_pool, v_pool, block_table, seq_lens, tasks, split_offsets,
                      num_partial_slots: int, scale: float, out, lse=None, stream=None,
                      k_scale: float = 1.0, v_scale: float = 1.0):
    """pkv_decode on the library's static workspace (no workspace argument, no
    allocation); see pkv_decode_static in include/pkv.h."""
    args = _decode_args(q, k_pool, v_pool, block_table, seq_lens, tasks, split_offsets,
                        num_partial_slots, scale, out, None, lse, stream, k_scale, v_scale)
    _check(_load().pkv_decode_static(*args), "pkv_decode_static")


def pkv_decode_splits(q, k_pool, v_pool, block_table, seq_lens, tasks, split_offsets,
                      num_partial_slots: int, scale: float, out, workspace, lse=None, stream=None,
                      k_scale: float = 1.0, v_scale: float = 1.0):
    """Enqueue the decode kernel only; see pkv_decode_splits in include/pkv.h."""
    args = _decode_args(q, k_pool, v_pool, block_table, seq_lens, tasks, split_offsets,
                        num_partial_slots, scale, out, workspace, lse, stream, k_scale, v_scale)
    _check(_load().pkv_decode_splits(*args), "pkv_decode_splits")


def pkv_merge(split_offsets, num_partial_slots: int, Hkv: int, out, workspace, lse=None,
              stream=None):
    """Enqueue the merge kernel only; see pkv_merge in include/pkv.h."""
    import torch
    code, edt = _elem_dtype(out)
    B, Hq, D = out.shape
    if split_offsets.shape != (B + 1,):
        raise ValueError("split_offsets must be [B+1]")
    if lse is not None and tuple(lse.shape) != (B, Hq):
        raise ValueError("lse must be [B, Hq]")
    _check(_load().pkv_merge(
        _dev(split_offsets, torch.int32, "split_offsets"), num_partial_slots, B, Hq, Hkv, D, code,
        _dev(out, edt, "out"),
        _dev(lse, torch.float32, "lse") if lse is not None else None,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream_ptr(stream)),
        "pkv_merge")


# --------------------------------------------------------------------------- device-side plan

def pkv_workspace_size_device_plan(B: int, Hq: int, Hkv: int, head_dim: int,
                                   max_splits: int) -> int:
    n = ctypes.c_size_t()
    _check(_load().pkv_workspace_size_device_plan(B, Hq, Hkv, head_dim, max_splits,
                                                  ctypes.byref(n)),
           "pkv_workspace_size_device_plan")
    return n.value


def pkv_decode_device_plan(q, k_pool, v_pool, block_table, seq_lens, scale: float, out,
                           workspace, max_splits: int, lse=None, mode: int = -1, param: int = 0,
                           params: Optional[pkv_policy_params] = None, num_cus: int = 0,
                           stream=None, k_scale: float = 1.0, v_scale: float = 1.0):
    """One step planned on the device; see pkv_decode_device_plan in include/pkv.h.
    seq_lens is a device tensor: nothing is read on the host."""
    import torch
    i32 = torch.int32
    code, f16, kvt = _dtypes(q, k_pool, v_pool, out)
    B, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_pool.shape
    if Dk != D or tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != (B, Hq, D):
        raise ValueError("shape mismatch between q, k_pool, v_pool and out")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    if lse is not None and tuple(lse.shape) != (B, Hq):
        raise ValueError("lse must be [B, Hq]")
    pp = ctypes.byref(params) if params is not None else None
    _check(_load().pkv_decode_device_plan(
        _dev(q, f16, "q"), _dev(k_pool, kvt, "k_pool"), _dev(v_pool, kvt, "v_pool"), num_pages,
        _dev(block_table, i32, "block_table"), block_table.shape[1], _dev(seq_lens, i32, "seq_lens"),
        B, Hq, Hkv, D, P, code, float(scale), float(k_scale), float(v_scale), mode, param,
        max_splits, pp, num_cus,
        _dev(out, f16, "out"), _dev(lse, torch.float32, "lse") if lse is not None else None,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream_ptr(stream)),
        "pkv_decode_device_plan")


def pkv_device_plan_read(workspace, B: int, Hq: int, Hkv: int, head_dim: int, max_splits: int,
                         stream=None):
    """(header dict, tasks [T,4], split_offsets [B+1]) of the last device plan."""
    import torch
    hdr = np.zeros(8, dtype=np.int32)
    offs = np.zeros(B + 1, dtype=np.int32)
    cap = Hkv * B * max_splits
    tasks = np.zeros((max(cap, 1), 4), dtype=np.int32)
    _check(_load().pkv_device_plan_read(
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), B, Hq, Hkv, head_dim,
        max_splits, hdr.ctypes.data_as(_i32p), _ptr(offs), _ptr(tasks), cap, _stream_ptr(stream)),
        "pkv_device_plan_read")
    keys = ("num_tasks", "fused", "mode", "param", "num_partial_slots", "max_splits", "row_flagged")
    return dict(zip(keys, (int(x) for x in hdr[:7]))), tasks[:hdr[0]].copy(), offs


# --------------------------------------------------------------------------- runner

def pkv_runner_create(num_cus: int = 0, params: Optional[pkv_policy_params] = None,
                      ring_depth: int = 8) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    pp = ctypes.byref(params) if params is not None else None
    _check(_load().pkv_runner_create(num_cus, pp, ring_depth, ctypes.byref(h)), "pkv_runner_create")
    return h


def pkv_runner_step(runner, args: pkv_step_args) -> int:
    """Run one step (see pkv_runner_step in include/pkv.h); returns the status
    (PKV_OK or PKV_ERR_BUFFER_TOO_SMALL), raising on any other error."""
    st = _load().pkv_runner_step(runner, ctypes.byref(args))
    if st not in (PKV_OK, PKV_ERR_BUFFER_TOO_SMALL):
        raise PkvError(st, "pkv_runner_step")
    return st


def pkv_runner_destroy(runner):
    _check(_load().pkv_runner_destroy(runner), "pkv_runner_destroy")


def pkv_runner_last_plan(runner):
    """Copies of the plan the last step's kernels read: (tasks [T,4], split_offsets [B+1])."""
    offs, tasks = ctypes.c_void_p(), ctypes.c_void_p()
    T, B = ctypes.c_int64(), ctypes.c_int32()
    _check(_load().pkv_runner_last_plan(runner, ctypes.byref(offs), ctypes.byref(tasks),
                                        ctypes.byref(T), ctypes.byref(B)), "pkv_runner_last_plan")
    o = np.ctypeslib.as_array(ctypes.cast(offs, _i32p), shape=(B.value + 1,)).copy()
    t = np.ctypeslib.as_array(ctypes.cast(tasks, _i32p), shape=(max(T.value, 1) * 4,))
    return t[:4 * T.value].reshape(T.value, 4).copy(), o


# --------------------------------------------------------------------------- plan / decode

class Plan:
    """A step's schedule: (mode, param), the compact task list and split
    offsets on the host (numpy) and on the device (int32 tensors), the number
    of partial-state slots and the deepest row's split count."""

    def __init__(self, mode, param, tasks, split_offsets, num_partial_slots, device):
        import torch
        self.mode, self.param = int(mode), int(param)
        self.tasks_host, self.offsets_host = tasks, split_offsets
        self.num_partial_slots = int(num_partial_slots)
        self.max_splits = int(np.max(np.diff(split_offsets))) if len(split_offsets) > 1 else 0
        self.tasks = torch.from_numpy(np.ascontiguousarray(tasks)).to(device)
        self.split_offsets = torch.from_numpy(np.ascontiguousarray(split_offsets)).to(device)

    @property
    def num_tasks(self) -> int:
        return len(self.tasks_host)


def plan(seq_lens, Hkv: int, max_pages_per_row: int, mode: Optional[int] = None,
         param: Optional[int] = None, num_cus: Optional[int] = None, head_dim: int = 128,
         dtype: int = PKV_DTYPE_F16, block_table=None, num_pages: int = 0,
         params: Optional[pkv_policy_params] = None, device="cuda") -> Plan:
    """Policy (when mode is None) and task list for host lengths ``seq_lens``:
    pkv_policy then pkv_plan (optionally checking a host block table), with
    the plan copied to ``device``."""
    import torch
    if mode is None:
        if num_cus is None:
            num_cus = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
        fp8 = dtype in (PKV_DTYPE_F16_KV_FP8, PKV_DTYPE_BF16_KV_FP8)
        mode, param = pkv_policy(seq_lens, Hkv, num_cus, params,
                                 head_dim=head_dim // 2 if fp8 else head_dim)
    tasks, offs, slots = pkv_plan(seq_lens, Hkv, max_pages_per_row, mode, param,
                                  block_table=block_table, num_pages=num_pages)
    return Plan(mode, param, tasks, offs, slots, device)


def decode(q, k_pool, v_pool, block_table, seq_lens, plan: Plan, scale: Optional[float] = None,
           out=None, lse=None, workspace=None, two_launch: Optional[bool] = None, stream=None,
           k_scale: float = 1.0, v_scale: float = 1.0,
           params: Optional[pkv_policy_params] = None):
    """One decode step on a plan: pkv_decode (merge fused), or
    pkv_decode_splits then pkv_merge when ``two_launch`` (None: the policy's
    rule: the deepest row has more than fuse_max_splits splits and the (row,
    KV head) groups times those splits exceed fuse_max_group_splits).  ``workspace`` (uint8,
    >= pkv_workspace_size, zeroed once by pkv_workspace_init) is made here
    when not given.  Returns (out, lse)."""
    import torch
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.zeros(pkv_workspace_size(plan.num_partial_slots, Hq, D),
                                dtype=torch.uint8, device=q.device)
        pkv_workspace_init(workspace, stream)
    if two_launch is None:
        p = params if params is not None else pkv_policy_defaults()
        groups = k_pool.shape[1] * int(np.count_nonzero(np.diff(plan.offsets_host)))
        two_launch = (plan.max_splits > p.fuse_max_splits and
                      groups * plan.max_splits > p.fuse_max_group_splits)
    args = (q, k_pool, v_pool, block_table, seq_lens, plan.tasks, plan.split_offsets,
            plan.num_partial_slots, scale, out, workspace)
    if two_launch:
        pkv_decode_splits(*args, lse=lse, stream=stream, k_scale=k_scale, v_scale=v_scale)
        pkv_merge(plan.split_offsets, plan.num_partial_slots, k_pool.shape[1], out, workspace,
                  lse=lse, stream=stream)
    else:
        pkv_decode(*args, lse=lse, stream=stream, k_scale=k_scale, v_scale=v_scale)
    return out, lse


class PagedDecoder:
    """Decode steps through the native runner: one library call per step runs
    policy -> host plan -> decode kernel (-> merge kernel in the two-launch
    form) on the given stream; the kernels read a new plan from the runner's
    pinned memory and a repeated one from its device copy.

    The decoder owns the workspace (a torch allocation, grown on demand) and a
    runner, whose pinned plan ring the kernels read in place.  The argument
    block is built once.  A step only rewrites the fields that change.
    """

    def __init__(self, Hq: int, Hkv: int, head_dim: int, max_batch: int, max_pages_per_row: int,
                 device=None, num_cus: Optional[int] = None, ring: int = 8,
                 policy_params: Optional[pkv_policy_params] = None):
        import torch
        self.Hq, self.Hkv, self.D = Hq, Hkv, head_dim
        self.max_pages = max_pages_per_row
        self.device = torch.device("cuda") if device is None else torch.device(device)
        if num_cus is None:
            num_cus = torch.cuda.get_device_properties(self.device).multi_processor_count
        self.num_cus = num_cus
        self.runner = pkv_runner_create(num_cus, policy_params, ring)
        self.workspace = torch.zeros(WORKSPACE_HEADER_BYTES, dtype=torch.uint8, device=self.device)
        pkv_workspace_init(self.workspace)
        self._seq_host = None
        a = pkv_step_args()
        a.Hq, a.Hkv, a.head_dim, a.page_size = Hq, Hkv, head_dim, PAGE_SIZE
        a.max_pages_per_row = max_pages_per_row
        self.args = a
        self._bind_buffers()
        self.last = None

    def _bind_buffers(self):
        a = self.args
        a.workspace = self.workspace.data_ptr()
        a.workspace_bytes = self.workspace.numel()

    def __del__(self):
        try:
            if getattr(self, "runner", None):
                pkv_runner_destroy(self.runner)
                self.runner = None
        except Exception:
            pass

    def set_inputs(self, q, k_pool, v_pool, block_table, seq_lens, seq_lens_h, scale: float,
                   out, lse=None, k_scale: float = 1.0, v_scale: float = 1.0):
        """Bind the tensors of the next steps (checked once here)."""
        import torch
        B, Hq, D = q.shape
        if (Hq, D) != (self.Hq, self.D) or k_pool.shape[1:] != (self.Hkv, PAGE_SIZE, D):
            raise ValueError("q / k_pool shape does not match the decoder")
        if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != (B, Hq, D):
            raise ValueError("shape mismatch between k_pool, v_pool, q and out")
        if tuple(block_table.shape) != (B, self.max_pages) or tuple(seq_lens.shape) != (B,):
            raise ValueError("block_table must be [B, max_pages_per_row] and seq_lens [B]")
        if lse is not None and tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
        a = self.args
        code, edt, kvt = _dtypes(q, k_pool, v_pool, out)
        a.dtype = code
        a.q = _dev(q, edt, "q").value
        a.k_pool = _dev(k_pool, kvt, "k_pool").value
        a.v_pool = _dev(v_pool, kvt, "v_pool").value
        a.num_pages = k_pool.shape[0]
        a.block_table = _dev(block_table, torch.int32, "block_table").value
        a.seq_lens = _dev(seq_lens, torch.int32, "seq_lens").value
        a.out = _dev(out, edt, "out").value
        a.lse = _dev(lse, torch.float32, "lse").value if lse is not None else None
        a.scale = float(scale)
        a.k_scale = float(k_scale)
        a.v_scale = float(v_scale)
        self._seq_host = np.ascontiguousarray(seq_lens_h, dtype=np.int32)
        a.seq_lens_host = self._seq_host.ctypes.data
        a.B = B
        self._tensors = (q, k_pool, v_pool, block_table, seq_lens, out, lse)

    def run(self, mode: Optional[int] = None, param: Optional[int] = None, stream=None,
            events=None, two_launch: Optional[bool] = None):
        """Enqueue one step on the bound inputs.  ``events`` = (before, after)
        torch.cuda.Event pair that takes the decode kernel's start and end
        timestamps (either may be None), or None.  ``two_launch``: True =
        separate merge kernel, False = fused single launch, None = the
        policy's rule (fuse_max_splits, fuse_max_group_splits)."""
        import torch
        a = self.args
        a.two_launch = -1 if two_launch is None else (1 if two_launch else 0)
        a.mode = -1 if mode is None else mode
        a.param = 0 if param is None else param
        a.stream = current_stream_ptr() if stream is None else stream.cuda_stream
        if events is not None:
            a.event_before_decode = None if events[0] is None else events[0].cuda_event
            a.event_after_decode = None if events[1] is None else events[1].cuda_event
        else:
            a.event_before_decode = None
            a.event_after_decode = None
        while pkv_runner_step(self.runner, a) == PKV_ERR_BUFFER_TOO_SMALL:
            step_stream = torch.cuda.current_stream() if stream is None else stream
            # Replace the workspace: every kernel that uses the old one is
            # queued on a stream of earlier steps (this one or the current
            # stream), so wait for both before torch may reuse it; the new
            # one is zeroed and initialised on the current stream, and
            # waited for, before any step on `step_stream` uses it.
            step_stream.synchronize()
            torch.cuda.current_stream().synchronize()
            if a.workspace_bytes_needed > a.workspace_bytes:
                self.workspace = torch.zeros(a.workspace_bytes_needed * 5 // 4 + 256,
                                             dtype=torch.uint8, device=self.device)
                pkv_workspace_init(self.workspace)
                torch.cuda.current_stream().synchronize()
            self._bind_buffers()
        self.last = (a.chosen_mode, a.chosen_param, a.num_tasks, a.num_partial_slots, a.B,
                     a.chosen_two_launch)
        return self.last

    def step(self, q, k_pool, v_pool, block_table, seq_lens, seq_lens_h, scale: float, out=None,
             lse=None, mode=None, param=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        self.set_inputs(q, k_pool, v_pool, block_table, seq_lens, seq_lens_h, scale, out, lse)
        self.run(mode, param)
        return out

    def plan_arrays(self):
        """The plan the last step's kernels read: (tasks [T,4], split_offsets [B+1])."""
        return pkv_runner_last_plan(self.runner)

    def error_flags(self) -> int:
        return pkv_workspace_error_flags(self.workspace)
