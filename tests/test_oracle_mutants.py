"""The pins must catch plausible mistakes.

Each mutant below is a copy of the oracle's ``attend`` with one planted
mistake (on the CPU, in oracle code only).  For every mutant at least one pin
of ``tests/pins.py`` must fail.
"""
import math

import numpy as np
import pytest

from tests import pins


def _make(mutation):
    def attend(q, k_pool, v_pool, block_table, seq_lens, scale, page_size=16):
        q = np.asarray(q)
        B, Hq, D = q.shape
        Hkv = k_pool.shape[1]
        G = Hq // Hkv
        out = np.zeros((B, Hq, D))
        lse = np.full((B, Hq), -np.inf)
        for b in range(B):
            N = int(seq_lens[b])
            if mutation == "read_one_more":
                N = N + 1
            if N == 0:
                continue
            t = np.arange(N)
            if mutation == "slot_from_page_index":
                pages = block_table[b, t // page_size]
                slots = (t // page_size) % page_size
            elif mutation == "logical_page_no_table":
                pages = t // page_size
                slots = t % page_size
            else:
                pages = block_table[b, t // page_size]
                slots = t % page_size
            pages = pages.astype(np.int64)
            for h in range(Hq):
                g = h % Hkv if mutation == "head_mod" else h // G
                K = k_pool[pages, g, slots, :].astype(np.float64)
                V = v_pool[pages, g, slots, :].astype(np.float64)
                if mutation == "k_for_v":
                    V = K
                sc = 1.0 if mutation == "no_scale" else scale
                s = sc * (K @ q[b, h].astype(np.float64))
                if mutation == "neg_scores":
                    s = -s
                m = s.max()
                w = np.exp(s - m)
                L = w.sum()
                if mutation == "no_normalise":
                    L = 1.0 if N > 1 else L
                out[b, h] = (w @ V) / L
                lse[b, h] = (math.log(L) if mutation == "lse_drops_max" else m + math.log(L))
        return out, lse
    return attend


MUTANTS = ["head_mod", "no_scale", "slot_from_page_index", "logical_page_no_table", "k_for_v",
           "neg_scores", "no_normalise", "lse_drops_max", "read_one_more"]


def test_unmutated_copy_passes_all_pins():
    for pin in pins.ALL_PINS:
        pin(_make(None))


@pytest.mark.parametrize("mutation", MUTANTS)
def test_pins_catch_mutant(mutation):
    attend = _make(mutation)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attend)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mutation}"
