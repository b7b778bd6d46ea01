"""Seeded synthetic inputs for paged GQA decode attention.

This module only draws inputs: sequence lengths, the shuffled page pool with its
block table, and fp16 N(0,1) query / key / value values.  It holds none of the
attention arithmetic, so both the float64 oracle and the HIP path may consume
what it produces.

Workload shapes follow the PersistentKV pages (arXiv 2606.26666): the abstracts
on the Lattice and fugumt.com pages fix FP16, page size 16, Hq=32, Hkv=8,
d=128, and the gist.science explainer ("Technische Samenvatting", section
"Evaluatieprotocol") names the synthetic trace families -- bucketed, bimodal,
uniform and Zipf-like -- and the calibration / held-out seeds 20260622 and
20260623 (section "Resultaten").

Draw order for a (config, seed) pair:
  1. lengths           numpy PCG64 ``default_rng(seed)``
  2. page permutation  same generator: ``permutation(pool_pages)``; row b owns
                       the next ceil(N_b/16) entries, in row order
  3. values            CPU: the same numpy generator, q then K then V, each
                       ``standard_normal(float32)`` rounded to fp16.
                       CUDA: ``torch.Generator('cuda').manual_seed(seed)``,
                       q then K then V, ``randn(float32)`` rounded to fp16.
The CPU and CUDA value streams differ for the same seed; lengths and the block
table are identical on both.  Finite garbage for unreferenced pages
(``fill="random"``) comes from a separate generator, so the referenced values
do not depend on the fill.

Poison: pool pages no row references and the tail slots t >= N_b of each
row's last page are filled with NaN (``fill="nan"``), and unused block-table
entries hold -1, so any read past a row's true length shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, Optional, Sequence

import numpy as np

PAGE_SIZE = 16

CALIBRATION_SEED = 20260622
HELD_OUT_SEEDS = (20260623, 20260624, 20260625, 20260626, 20260627)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    max_pages_per_row: int
    pool_pages: int
    lengths: Callable[[np.random.Generator], np.ndarray]
    splits: Sequence[int] = ()
    page_size: int = PAGE_SIZE
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


def _fixed(n: int, B: int = 1):
    return lambda rng: np.full(B, n, dtype=np.int64)


def _bimodal(rng: np.random.Generator) -> np.ndarray:
    short = rng.integers(256, 1025, size=4)
    long_ = rng.integers(12288, 16385, size=4)
    return rng.permutation(np.concatenate([short, long_]))


def _zipf(rng: np.random.Generator) -> np.ndarray:
    return np.minimum(32768, 512 * rng.zipf(1.2, size=8))


def _uniform8(rng: np.random.Generator) -> np.ndarray:
    return rng.integers(1024, 32769, size=8)


def _uniform64(rng: np.random.Generator) -> np.ndarray:
    return rng.integers(4096, 65537, size=64)


def _bucketed1(rng: np.random.Generator) -> np.ndarray:
    # one long-context row whose length falls in a power-of-two bucket
    bucket = int(rng.choice([8192, 16384, 32768, 65536]))
    return np.array([rng.integers(bucket // 2 + 1, bucket + 1)])


def _bimodal4(rng: np.random.Generator) -> np.ndarray:
    short = rng.integers(256, 1025, size=2)
    long_ = rng.integers(12288, 16385, size=2)
    return rng.permutation(np.concatenate([short, long_]))


def _uniform32(rng: np.random.Generator) -> np.ndarray:
    return rng.integers(1024, 32769, size=32)


CONFIGS: Dict[str, Config] = {
    c.name: c
    for c in [
        Config("tiny", B=1, Hq=4, Hkv=1, D=64, max_pages_per_row=16, pool_pages=64,
               lengths=_fixed(256), splits=(1, 4),
               description="B=1 Hq4 Hkv1 d64, N=256 (16 pages) in a 64-page pool"),
        Config("b1", B=1, Hq=32, Hkv=8, D=128, max_pages_per_row=2048, pool_pages=4096,
               lengths=_fixed(32768), splits=(8, 16, 32, 64),
               description="B=1 long context, N=32768 (2048 pages) in a 4096-page pool"),
        Config("b8_bimodal", B=8, Hq=32, Hkv=8, D=128, max_pages_per_row=1024,
               pool_pages=2 * 8 * 1024, lengths=_bimodal,
               description="B=8, 4 rows U[256,1024] + 4 rows U[12288,16384], shuffled"),
        Config("b8_zipf", B=8, Hq=32, Hkv=8, D=128, max_pages_per_row=2048,
               pool_pages=2 * 8 * 2048, lengths=_zipf,
               description="B=8, N=min(32768, 512*k), k~Zipf(1.2)"),
        Config("b8_uniform", B=8, Hq=32, Hkv=8, D=128, max_pages_per_row=2048,
               pool_pages=2 * 8 * 2048, lengths=_uniform8,
               description="B=8, N~U[1024,32768]"),
        Config("b64", B=64, Hq=32, Hkv=8, D=128, max_pages_per_row=4096,
               pool_pages=2 * 64 * 4096, lengths=_uniform64,
               description="B=64, N~U[4096,65536], 34.4 GB K+V pool"),
        # traces of the policy calibration protocol
        Config("b1_bucketed", B=1, Hq=32, Hkv=8, D=128, max_pages_per_row=4096,
               pool_pages=8192, lengths=_bucketed1,
               description="B=1, bucket in {8K,16K,32K,64K}, N~U(bucket/2, bucket]"),
        Config("b4_bimodal", B=4, Hq=32, Hkv=8, D=128, max_pages_per_row=1024,
               pool_pages=2 * 4 * 1024, lengths=_bimodal4,
               description="B=4, 2 rows U[256,1024] + 2 rows U[12288,16384], shuffled"),
        Config("b32_uniform", B=32, Hq=32, Hkv=8, D=128, max_pages_per_row=2048,
               pool_pages=2 * 32 * 2048, lengths=_uniform32,
               description="B=32, N~U[1024,32768] (B*Hkv = one task per CU unsplit)"),
    ]
}


@dataclasses.dataclass
class Workload:
    """One batch of decode inputs.

    q         [B, Hq, D]                    fp16
    k_pool    [pool_pages, Hkv, 16, D]      fp16
    v_pool    [pool_pages, Hkv, 16, D]      fp16
    block_table [B, max_pages_per_row]      int32, -1 where unused
    seq_lens  [B]                           int32
    Tensors are torch tensors on ``device``; ``seq_lens_np`` and
    ``block_table_np`` are host copies.
    """
    cfg: Config
    seed: int
    seq_lens_np: np.ndarray
    block_table_np: np.ndarray
    q: "object"
    k_pool: "object"
    v_pool: "object"
    block_table: "object"
    seq_lens: "object"

    @property
    def scale(self) -> float:
        return self.cfg.scale

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V the batch attends over: sum_b N_b*Hkv*D*2*e, with e
        the bytes of one pool element (2 for fp16 / bf16, 1 for fp8)."""
        e = self.k_pool.element_size() if hasattr(self.k_pool, "element_size") else 2
        return int(self.seq_lens_np.astype(np.int64).sum()) * self.cfg.Hkv * self.cfg.D * 2 * e


def make_lengths(cfg: Config, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return cfg.lengths(rng).astype(np.int32)


def build_block_table(cfg: Config, seq_lens: np.ndarray, rng: np.random.Generator,
                      pool_pages: Optional[int] = None) -> np.ndarray:
    """Row b owns the next ceil(N_b/16) entries of a permutation of the pool."""
    pool_pages = cfg.pool_pages if pool_pages is None else pool_pages
    n_pages = (seq_lens.astype(np.int64) + cfg.page_size - 1) // cfg.page_size
    if int(n_pages.max(initial=0)) > cfg.max_pages_per_row:
        raise ValueError("a row needs more pages than max_pages_per_row")
    if int(n_pages.sum()) > pool_pages:
        raise ValueError("pool too small for the batch")
    perm = rng.permutation(pool_pages)
    bt = np.full((len(seq_lens), cfg.max_pages_per_row), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[off:off + n]
        off += int(n)
    return bt


def make_workload(name_or_cfg, seed: int, device: str = "cpu", fill: str = "nan",
                  seq_lens: Optional[Sequence[int]] = None,
                  pool_pages: Optional[int] = None, dtype: str = "f16") -> Workload:
    """Draw one batch.  ``seq_lens`` overrides the config's length draw (edge cases).

    fill: what unreferenced pool pages and tail slots hold: "nan", "random" or "zero".
    dtype: "f16", or (device workloads only) "bf16": the same float32 draws
    rounded to bfloat16 instead of fp16; "fp8": q fp16 and K / V pools of fp8
    E4M3 codes (torch.float8_e4m3fn), the float32 draws rounded to E4M3;
    "bf16_fp8": the same with q in bfloat16.  Poison fills of fp8 pools use
    the NaN code 0x7F.
    """
    import torch

    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    rng = np.random.default_rng(seed)
    lens = cfg.lengths(rng) if seq_lens is None else np.asarray(seq_lens)
    lens = lens.astype(np.int32)
    pool = cfg.pool_pages if pool_pages is None else pool_pages
    bt = build_block_table(cfg, lens, rng, pool)
    P = cfg.page_size
    n_pages = (lens.astype(np.int64) + P - 1) // P
    used = np.concatenate([bt[b, :n] for b, n in enumerate(n_pages)]) if n_pages.sum() else \
        np.zeros(0, dtype=np.int32)
    pshape = (pool, cfg.Hkv, P, cfg.D)

    if dtype not in ("f16", "bf16", "fp8", "bf16_fp8"):
        raise ValueError(dtype)
    if device == "cpu" and dtype != "f16":
        raise ValueError("bf16 and fp8 workloads are drawn on the device only")
    if device == "cpu":
        fill_rng = np.random.default_rng([seed, 1])
        q = rng.standard_normal((len(lens), cfg.Hq, cfg.D), dtype=np.float32).astype(np.float16)
        pools = []
        for _ in range(2):
            vals = rng.standard_normal((len(used), cfg.Hkv, P, cfg.D), dtype=np.float32)
            vals = vals.astype(np.float16)
            if fill == "nan":
                arr = np.full(pshape, np.nan, dtype=np.float16)
            elif fill == "zero":
                arr = np.zeros(pshape, dtype=np.float16)
            elif fill == "random":
                arr = fill_rng.standard_normal(pshape, dtype=np.float32).astype(np.float16)
            else:
                raise ValueError(fill)
            arr[used] = vals
            pools.append(arr)
        k_np, v_np = pools
        _poison_tails(k_np, v_np, bt, lens, P, fill, rng)
        q_t = torch.from_numpy(q)
        k_t = torch.from_numpy(k_np)
        v_t = torch.from_numpy(v_np)
        bt_t = torch.from_numpy(bt.copy())
        sl_t = torch.from_numpy(lens.copy())
    else:
        dev = torch.device(device)
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        fill_gen = torch.Generator(device=dev)
        fill_gen.manual_seed(seed + 7919)
        edt = torch.bfloat16 if dtype in ("bf16", "bf16_fp8") else torch.float16
        fp8 = dtype in ("fp8", "bf16_fp8")
        # pools of fp8 codes are built as uint8 (fills, copies) and viewed as
        # float8_e4m3fn at the end; the draws are rounded by torch's conversion
        pdt = torch.uint8 if fp8 else edt

        def to_pool(x):
            return x.to(torch.float8_e4m3fn).view(torch.uint8) if fp8 else x.to(edt)

        q_t = torch.randn((len(lens), cfg.Hq, cfg.D), generator=gen, device=dev,
                          dtype=torch.float32).to(edt)
        used_t = torch.from_numpy(used.astype(np.int64)).to(dev)
        pools = []
        nan_val = 0x7F if fp8 else float("nan")
        for _ in range(2):
            if fill == "nan":
                arr = torch.full(pshape, nan_val, dtype=pdt, device=dev)
            elif fill == "zero":
                arr = torch.zeros(pshape, dtype=pdt, device=dev)
            elif fill == "random":
                arr = torch.empty(pshape, dtype=pdt, device=dev)
                _randn_fill(arr, fill_gen, to_pool)
            else:
                raise ValueError(fill)
            # referenced pages, generated in chunks to bound the fp32 temporary
            chunk = max(1, (1 << 28) // (cfg.Hkv * P * cfg.D))
            for i in range(0, len(used), chunk):
                idx = used_t[i:i + chunk]
                vals = to_pool(torch.randn((idx.numel(), cfg.Hkv, P, cfg.D), generator=gen,
                                           device=dev, dtype=torch.float32))
                arr.index_copy_(0, idx, vals)
                del vals
            pools.append(arr)
        k_t, v_t = pools
        if fill != "random":
            tail_val = nan_val if fill == "nan" else 0
            for b, n in enumerate(lens):
                r = int(n) % P
                if n > 0 and r:
                    last = int(bt[b, (int(n) - 1) // P])
                    k_t[last, :, r:, :] = tail_val
                    v_t[last, :, r:, :] = tail_val
        if fp8:
            k_t = k_t.view(torch.float8_e4m3fn)
            v_t = v_t.view(torch.float8_e4m3fn)
        bt_t = torch.from_numpy(bt.copy()).to(dev)
        sl_t = torch.from_numpy(lens.copy()).to(dev)
    return Workload(cfg=cfg, seed=seed, seq_lens_np=lens, block_table_np=bt, q=q_t,
                    k_pool=k_t, v_pool=v_t, block_table=bt_t, seq_lens=sl_t)


def _randn_fill(arr, gen, convert=None):
    import torch
    flat = arr.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        x = torch.randn(n, generator=gen, device=arr.device, dtype=torch.float32)
        flat[i:i + n] = convert(x) if convert is not None else x.to(arr.dtype)


def _poison_tails(k, v, bt, lens, P, fill, rng):
    if fill == "random":
        return
    val = np.float16(np.nan) if fill == "nan" else np.float16(0)
    for b, n in enumerate(lens):
        r = int(n) % P
        if n > 0 and r:
            last = int(bt[b, (int(n) - 1) // P])
            k[last, :, r:, :] = val
            v[last, :, r:, :] = val


def relabel_pages(wl_np: dict, rng: np.random.Generator) -> dict:
    """Return the same batch with pool pages relabelled by a random permutation.

    ``wl_np`` holds numpy arrays k_pool, v_pool, block_table.  Page p moves to
    slot perm[p]; block-table entries are rewritten to follow (-1 stays -1).
    """
    k, v, bt = wl_np["k_pool"], wl_np["v_pool"], wl_np["block_table"]
    perm = rng.permutation(k.shape[0])
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    bt2 = np.where(bt >= 0, perm[np.clip(bt, 0, None)], -1).astype(bt.dtype)
    out = dict(wl_np)
    out.update(k_pool=k2, v_pool=v2, block_table=bt2)
    return out


def compact_rows(q, k_pool, v_pool, block_table, seq_lens, rows, page_size=PAGE_SIZE):
    """Copy out only the pages of ``rows`` (host numpy), renumbered densely.

    Used to check sampled rows of very large batches without moving the whole
    pool to the host.  Accepts torch tensors (any device) or numpy arrays.
    Returns numpy q, k_pool, v_pool, block_table, seq_lens for those rows.
    """
    import torch

    rows = list(rows)
    bt = block_table.cpu().numpy() if hasattr(block_table, "cpu") else np.asarray(block_table)
    sl = seq_lens.cpu().numpy() if hasattr(seq_lens, "cpu") else np.asarray(seq_lens)
    bt = bt[rows]
    sl = sl[rows]
    n = (sl.astype(np.int64) + page_size - 1) // page_size
    used = np.concatenate([bt[i, :n[i]] for i in range(len(rows))]) if n.sum() else \
        np.zeros(0, np.int64)
    uniq, inv = np.unique(used, return_inverse=True)
    new_bt = np.full_like(bt, -1)
    off = 0
    for i in range(len(rows)):
        new_bt[i, :n[i]] = inv[off:off + n[i]]
        off += int(n[i])

    def take(pool):
        if isinstance(pool, np.ndarray):
            return pool[uniq]
        idx = torch.from_numpy(uniq.astype(np.int64)).to(pool.device)
        if pool.dtype == torch.float8_e4m3fn:   # E4M3 codes, decoded by the reader
            return pool.view(torch.uint8).index_select(0, idx).cpu().numpy()
        sel = pool.index_select(0, idx)
        if sel.dtype == torch.bfloat16:       # numpy has no bfloat16: widen exactly
            sel = sel.float()
        return sel.cpu().numpy()

    if hasattr(q, "cpu"):
        qn = (q.float() if q.dtype == torch.bfloat16 else q).cpu().numpy()
    else:
        qn = np.asarray(q)
    return qn[rows], take(k_pool), take(v_pool), new_bt, sl
