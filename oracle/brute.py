"""Pure-Python loop version of the decode definition, for tiny shapes only.

Test infrastructure (see the oracle package doc).  Written without numpy so it
can pin ``oracle.ref.attend``: every product and sum is an explicit loop, sums
use ``math.fsum`` (exactly rounded), exponentials use ``math.exp``.

Definition followed: PersistentKV (arXiv 2606.26666), gist.science explainer,
"Technische Samenvatting" > Methodologie > "1. Native Block-Table Decode
Engine" (GQA with G = Hq/Hkv query heads per KV head, decode over the native
block table) with the readings listed in the package doc.
"""
from __future__ import annotations

import math


def attend_loops(q, k_pool, v_pool, block_table, seq_lens, scale, page_size=16):
    """q[b][h][j], pools[page][g][slot][j], block_table[b][i], seq_lens[b] as
    nested sequences of Python numbers.  Returns (out, lse) as nested lists."""
    B = len(q)
    Hq = len(q[0])
    D = len(q[0][0])
    Hkv = len(k_pool[0])
    G = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    lse = [[-math.inf] * Hq for _ in range(B)]
    for b in range(B):
        N = int(seq_lens[b])
        if N == 0:
            continue
        for h in range(Hq):
            g = h // G
            scores = []
            for t in range(N):
                page = int(block_table[b][t // page_size])
                slot = t % page_size
                dot = math.fsum(float(q[b][h][j]) * float(k_pool[page][g][slot][j])
                                for j in range(D))
                scores.append(scale * dot)
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            L = math.fsum(w)
            for j in range(D):
                acc = []
                for t in range(N):
                    page = int(block_table[b][t // page_size])
                    acc.append(w[t] * float(v_pool[page][g][t % page_size][j]))
                out[b][h][j] = math.fsum(acc) / L
            lse[b][h] = m + math.log(L)
    return out, lse


def tasks_by_walking(seq_lens, Hkv, page_size, chunk_of_row):
    """Task list built by walking every (row, KV head, page) one at a time and
    opening a new task every ``chunk_of_row(b, n_b)`` pages.  Independent of
    the closed-form construction in ``oracle.ref.plan_tasks``."""
    tasks = []
    for b, N in enumerate(seq_lens):
        N = int(N)
        n = 0
        while n * page_size < N:
            n += 1
        if n == 0:
            continue
        c = chunk_of_row(b, n)
        for g in range(Hkv):
            s = -1
            for p in range(n):
                if p % c == 0:
                    s += 1
                    tasks.append([b, g, s, c])
    return tasks
