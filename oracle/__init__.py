"""Float64 CPU oracle for paged GQA decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything in this package.  The product
path (the HIP library and its Python binding) never does, and shares no code
with it: no kernels, helpers, constants or tables.

What it computes is fixed by the PersistentKV pages (arXiv 2606.26666):
  * GQA decode: G = Hq/Hkv query heads share one KV head, one new query token
    per row (gist.science explainer, "Technische Samenvatting" > Methodologie >
    "1. Native Block-Table Decode Engine"; Lattice and fugumt.com abstracts).
  * The KV cache is read in place through a per-row block table of 16-token
    pages (same section, item "Layout"; abstracts: page size 16).
  * Sequence splitting into disjoint ranges with an exact merge of partial
    online-softmax states, row-local bounds from the true lengths, and a
    compact list of non-empty (row, KV head, split) tasks (same section, items
    "Sequentie Splitting", "Row-Local Bounds", "Compact Workqueue").
  The schedule (split count, chunk) only decides how the same result is
    computed, so it has no place here: the task list is computed for any
    given mode and parameter, and every schedule must reach ``attend``'s
    result.  (The library's scheduling policy is checked against the pages'
    mode rule and against a second implementation of its documented model in
    the tests, not against this package.)

fp8 KV pools (beyond the pages, which use FP16): the values are the OCP E4M3
codes of the pool times a per-tensor scale (``e4m3_decode``, ``kv_values``),
decoded from the format's published definition.

Readings taken where the pages are silent:
  scale = 1/sqrt(d); query head h reads KV head floor(h/G); token t of a row
  lives in page block_table[b, t // 16] at slot t % 16; K and V pools are
  [num_pages, Hkv, 16, d]; a row with N_b = 0 yields out = 0, lse = -inf.

Pins: every function here is checked against something other than itself in
``tests/test_oracle_pins.py`` (brute force, closed forms, a library special
case, invariances).
"""
from .ref import (  # noqa: F401
    MODE_SPLIT,
    MODE_WORKQUEUE,
    attend,
    e4m3_decode,
    kv_values,
    merge_states,
    partial_state,
    plan_tasks,
    split_merge,
)
