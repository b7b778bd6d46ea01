"""Float64 reference for paged GQA decode (test infrastructure only; see package doc).

Source: PersistentKV, arXiv 2606.26666.  Section names below refer to the
gist.science explainer's "Technische Samenvatting" (technical summary) unless
another page is named.
"""
from __future__ import annotations

import math

import numpy as np

MODE_SPLIT = 0
MODE_WORKQUEUE = 1


# ---------------------------------------------------------------------------
# dense definition
# ---------------------------------------------------------------------------

def _row_tokens(block_table, b, t0, t1, page_size):
    """Physical (page, slot) of logical tokens t0..t1-1 of row b.

    Methodologie > "Layout": decode runs over the native paged layout through
    the block table, without repacking pages into a contiguous tensor.
    Reading: token t sits in page block_table[b, t // page_size], slot
    t % page_size.
    """
    t = np.arange(t0, t1)
    return block_table[b, t // page_size].astype(np.int64), t % page_size


# ---------------------------------------------------------------------------
# fp8 KV values
# ---------------------------------------------------------------------------

def e4m3_decode(codes):
    """Value of OCP E4M3 codes ("e4m3fn"), float64.

    Definition: OCP 8-bit Floating Point Specification (OFP8), the E4M3
    format: 1 sign bit s, 4 exponent bits e with bias 7, 3 mantissa bits m;
    e > 0 is normal, (-1)^s 2^(e-7) (1 + m/8); e = 0 is subnormal,
    (-1)^s 2^-6 (m/8); there are no infinities, and e = 15 with m = 7 is
    NaN (so the largest finite magnitude is 2^8 * 1.75 = 448).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def kv_values(pool, kv_scale=1.0):
    """Dequantised values of a K or V pool, float64: kv_scale * x.

    A uint8 pool holds E4M3 codes (``e4m3_decode``); any other array holds
    the values themselves (fp16, or bf16 widened exactly to float32).  The
    scale is the per-tensor dequantisation factor of an fp8 cache (1 for
    fp16 / bf16).
    """
    a = np.asarray(pool)
    x = e4m3_decode(a) if a.dtype == np.uint8 else a.astype(np.float64)
    return x * float(kv_scale) if kv_scale != 1.0 else x


def attend(q, k_pool, v_pool, block_table, seq_lens, scale, page_size=16, k_scale=1.0,
           v_scale=1.0):
    """Single-query GQA attention of every row over its own paged KV.

    For row b, query head h, with G = Hq/Hkv and KV head g = floor(h/G)
    (Methodologie > "1. Native Block-Table Decode Engine": G query heads share
    one KV head; the head-to-group map floor(h/G) is the contiguous-group
    reading):
        s_t  = scale * <q[b,h], K_t>          t = 0..N_b-1
        out  = sum_t softmax(s)_t * V_t
        lse  = log sum_t exp(s_t)
    All arithmetic in float64 after exact upcast of the inputs; K_t and V_t
    are the dequantised values k_scale * K and v_scale * V (``kv_values``:
    uint8 pools are fp8 E4M3 codes).  N_b = 0 gives out = 0, lse = -inf.

    Shapes: q [B,Hq,D]; k_pool, v_pool [num_pages, Hkv, page_size, D];
    block_table [B, max_pages]; seq_lens [B].  Returns (out [B,Hq,D],
    lse [B,Hq]) as float64.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    k_pool = kv_values(k_pool, k_scale)
    v_pool = kv_values(v_pool, v_scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        N = int(seq_lens[b])
        if N == 0:
            continue
        pages, slots = _row_tokens(block_table, b, 0, N, page_size)
        for g in range(Hkv):
            K = k_pool[pages, g, slots, :].astype(np.float64)      # [N, D]
            V = v_pool[pages, g, slots, :].astype(np.float64)      # [N, D]
            for h in range(g * G, (g + 1) * G):
                s = scale * (K @ q[b, h].astype(np.float64))         # [N]
                m = s.max()
                w = np.exp(s - m)
                L = w.sum()
                out[b, h] = (w @ V) / L
                lse[b, h] = m + math.log(L)
    return out, lse


# ---------------------------------------------------------------------------
# task list
# ---------------------------------------------------------------------------

def plan_tasks(seq_lens, Hkv, page_size, mode, param):
    """Compact list of non-empty (row, KV head, split) tasks.

    Methodologie > "Row-Local Bounds": tile counts and split ranges come from
    each row's true length N_b, not a padded one.  "Sequentie Splitting": the
    sequence is cut into disjoint ranges.  "Compact Workqueue": only non-empty
    row-KV-head-split intervals are emitted, as a 1D list.

    Reading (the pages give no formula): with n_b = ceil(N_b/page_size) pages,
      split mode     (param = S): chunk c_b = ceil(n_b / S)
      workqueue mode (param = c): chunk c_b = c
      S_b = ceil(n_b / c_b)  (0 when N_b = 0)
    Split s of row b covers pages [s*c_b, min((s+1)*c_b, n_b)).  The record is
    (row, kv_head, split, c_b), ordered by row, then KV head, then split.
    split_offsets is the exclusive prefix sum of S_b (length B+1).

    Returns (tasks int32 [T,4], split_offsets int32 [B+1]).
    """
    if mode not in (MODE_SPLIT, MODE_WORKQUEUE):
        raise ValueError("unknown mode")
    if param < 1:
        raise ValueError("param must be >= 1")
    tasks = []
    offsets = [0]
    for b, N in enumerate(seq_lens):
        N = int(N)
        n = -(-N // page_size)
        if n == 0:
            offsets.append(offsets[-1])
            continue
        c = -(-n // param) if mode == MODE_SPLIT else int(param)
        S = -(-n // c)
        offsets.append(offsets[-1] + S)
        for g in range(Hkv):
            for s in range(S):
                tasks.append((b, g, s, c))
    t = np.array(tasks, dtype=np.int32).reshape(-1, 4)
    return t, np.array(offsets, dtype=np.int32)


# ---------------------------------------------------------------------------
# split + merge
# ---------------------------------------------------------------------------

def partial_state(q_heads, K, V, scale):
    """Online-softmax state of a token range for a group of query heads.

    "Sequentie Splitting": each split computes a partial online-softmax state.
    State per head: m = max_t s_t, l = sum_t exp(s_t - m),
    o = sum_t exp(s_t - m) V_t.  An empty range is the neutral state
    (m=-inf, l=0, o=0) ("Row-Local Bounds": empty splits write neutral states).
    q_heads [G,D], K/V [n,D] float64.  Returns m [G], l [G], o [G,D].
    """
    G, D = q_heads.shape
    if K.shape[0] == 0:
        return np.full(G, -np.inf), np.zeros(G), np.zeros((G, D))
    s = scale * (K @ q_heads.T).T                                  # [G, n]
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])
    return m, w.sum(axis=1), w @ V


def merge_states(m, l, o):
    """Exact log-sum-exp merge of S partial states of one query head.

    "Sequentie Splitting": a separate merge combines the split states exactly.
    M = max_s m_s, w_s = exp(m_s - M) (0 for neutral states),
    out = sum_s w_s o_s / sum_s w_s l_s, lse = M + log sum_s w_s l_s.
    All-neutral input gives out = 0, lse = -inf.
    m, l [S]; o [S,D].  Returns (out [D], lse).
    """
    m = np.asarray(m, dtype=np.float64)
    if m.size == 0 or np.all(np.isneginf(m)):
        return np.zeros(np.asarray(o).shape[-1]), -np.inf
    M = m.max()
    w = np.where(np.isneginf(m), 0.0, np.exp(m - M))
    L = (w * l).sum()
    return (w[:, None] * o).sum(axis=0) / L, M + math.log(L)


def split_merge(q, k_pool, v_pool, block_table, seq_lens, scale, tasks, split_offsets,
                page_size=16, extra_neutral=0, k_scale=1.0, v_scale=1.0):
    """Walk a task list, form each task's partial state, merge per (row, head).

    Task (b, g, s, c) covers tokens [s*c*P, min((s+1)*c*P, N_b)) of row b for
    KV head g and all G query heads of that group (the v1/v2 abstracts: work
    is mapped by KV-head group so one K/V tile serves the grouped query heads).
    ``extra_neutral`` appends that many neutral states to every merge.  The
    pools are read as in ``attend`` (``kv_values``).
    Returns (out [B,Hq,D], lse [B,Hq]) float64.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    k_pool = kv_values(k_pool, k_scale)
    v_pool = kv_values(v_pool, v_scale)
    nslots = int(split_offsets[-1])
    m = np.full((nslots, Hq), -np.inf)
    l = np.zeros((nslots, Hq))
    o = np.zeros((nslots, Hq, D))
    for b, g, s, c in np.asarray(tasks).reshape(-1, 4):
        N = int(seq_lens[b])
        t0 = int(s) * int(c) * page_size
        t1 = min((int(s) + 1) * int(c) * page_size, N)
        pages, slots = _row_tokens(block_table, b, t0, t1, page_size)
        K = k_pool[pages, g, slots, :].astype(np.float64)
        V = v_pool[pages, g, slots, :].astype(np.float64)
        slot = int(split_offsets[b]) + int(s)
        hs = slice(g * G, (g + 1) * G)
        m[slot, hs], l[slot, hs], o[slot, hs] = partial_state(
            q[b, hs].astype(np.float64), K, V, scale)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        sl = slice(int(split_offsets[b]), int(split_offsets[b + 1]))
        for h in range(Hq):
            mm, ll, oo = m[sl, h], l[sl, h], o[sl, h]
            if extra_neutral:
                mm = np.concatenate([mm, np.full(extra_neutral, -np.inf)])
                ll = np.concatenate([ll, np.zeros(extra_neutral)])
                oo = np.concatenate([oo, np.zeros((extra_neutral, D))])
            out[b, h], lse[b, h] = merge_states(mm, ll, oo)
    return out, lse
