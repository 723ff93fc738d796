"""CPU oracle for the KV write (recompute-scatter) step -- test infrastructure only.

Nothing in the product path may import, call or link this module; the tests,
the package smoke check and the benchmark's CPU-baseline leg may.

What the step does (AsymCache / Multi-Segment Attention paper): evicted KV
blocks are rebuilt on demand so that attention stays exact (abstract), and
the rebuilt blocks together with a prefill chunk's own K/V become ordinary
segments of the block-paged cache that Multi-Segment Attention then reads in
one launch (section 4.1, Figure 5 schematic).  Before that attention runs,
the freshly computed K and V rows have to be placed where the segment
descriptors say they live.

Reading taken (the pages do not spell out the write): token ``i`` of a fresh
segment ``(pos_start, len, bt_start, flags)`` whose rows start at ``src_row``
of the fresh arrays goes to pool block ``block_table[bt_start + i // 16]``,
slot ``i % 16``, for every kv head -- the same addressing the attention reads
with.  Slots no fresh token maps to keep their contents.  It is a pure copy,
so the result is exact (bit for bit) in any dtype.

Pins (``tests/test_kv_write_oracle.py``): literal slot placement of a hand
example, round trip through the attention oracle's gather, untouched slots
unchanged, and write-then-attend equal to plain causal attention.
"""
from __future__ import annotations

import numpy as np


def write_kv(K_pool, V_pool, k_src, v_src, segments, src_rows, block_table, block_size=16):
    """Return copies of ``K_pool``/``V_pool`` ([num_blocks, H_kv, bs, d], any
    dtype) with each fresh segment's rows of ``k_src``/``v_src``
    ([rows, H_kv, d]) written into its blocks."""
    K = np.array(K_pool, copy=True)
    V = np.array(V_pool, copy=True)
    bt = np.asarray(block_table)
    for seg, row0 in zip(segments, src_rows):
        length, bt_start = int(seg[1]), int(seg[2])
        if length == 0:
            continue
        i = np.arange(length)
        ids = bt[bt_start + i // block_size]
        slots = i % block_size
        rows = int(row0) + i
        K[ids, :, slots, :] = np.asarray(k_src)[rows]
        V[ids, :, slots, :] = np.asarray(v_src)[rows]
    return K, V
