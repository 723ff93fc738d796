"""fp64 CPU oracle for Multi-Segment Attention (MSA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module; it exists so that the tests, the package smoke check and the
benchmark's CPU baseline can check the HIP path against a plain, slow and
obviously correct statement of what MSA computes.

What MSA computes (AsymCache / Multi-Segment Attention paper):

* Eq. 1 (Figure 1 caption): ``A = Q K^T / sqrt(d_k)``, ``O = softmax(A) V``.
* Section 4.1 (Figure 4 caption): the KV context of a request may be made of
  several disjoint regions of the cache (e.g. both a cached prefix and a cached
  suffix), which one attention kernel must handle.
* Abstract: evicted blocks are rebuilt on demand so that outputs stay exact;
  so MSA's result is exactly attention over the gathered context.
* Eq. 5 (Figure 6 caption): the regions l1, q1, l2, q2 of a request keep their
  places in the sequence, so causality is decided by absolute token position,
  not by the order in which segments are gathered.

Readings taken where the pages are silent (each is stated again in the
design notes):

* scale defaults to ``1/sqrt(head_dim)`` (Eq. 1's d_k);
* causal visibility is ``k_pos <= q_pos`` (the diagonal is visible);
* kv head of q head ``h`` is ``h // (H_q / H_kv)`` (contiguous GQA groups);
* a row with no visible key has output 0 and log-sum-exp -inf;
* ``lse`` is the natural log of ``sum_j exp(scale * q . k_j)`` over visible keys.

Parity pins: brute force on tiny inputs, torch's fp64 scaled-dot-product
attention for the single-segment case, invariants (segment order, segment
split, position shift, gaps, NaN poison outside segments, row sums), closed
forms (q = 0, one visible key, constant V, GQA head probe) and the log-sum-exp
merge identity.  All live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import math

import numpy as np


def gather_context(segments, block_table, K_pool, V_pool, block_size=16):
    """Gather one sequence's keys, values and absolute key positions.

    Segments are taken in the order given (descriptor order, not position
    order): token ``i`` of segment ``(pos_start, len, bt_start, flags)`` sits in
    pool block ``block_table[bt_start + i // block_size]`` at slot
    ``i % block_size`` and has position ``pos_start + i``.

    Returns ``K [n, H_kv, d]``, ``V [n, H_kv, d]`` (float64) and ``pos [n]``.
    """
    ks, vs, ps = [], [], []
    for seg in segments:
        pos_start, length, bt_start = int(seg[0]), int(seg[1]), int(seg[2])
        if length == 0:
            continue
        i = np.arange(length)
        ids = np.asarray(block_table)[bt_start + i // block_size]
        slots = i % block_size
        ks.append(np.asarray(K_pool[ids, :, slots, :], dtype=np.float64))
        vs.append(np.asarray(V_pool[ids, :, slots, :], dtype=np.float64))
        ps.append(pos_start + i)
    if not ks:
        shape = (0,) + tuple(K_pool.shape[1:2]) + tuple(K_pool.shape[3:4])
        return np.zeros(shape), np.zeros(shape), np.zeros(0, dtype=np.int64)
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(ps).astype(np.int64)


def masked_softmax_attention(q, k, v, q_pos, k_pos, scale, causal=True, return_probs=False):
    """Eq. 1 with a position mask for one head.

    ``q [m, d]``, ``k [n, d]``, ``v [n, d]`` in float64.  Key ``j`` is visible
    to row ``i`` iff ``k_pos[j] <= q_pos[i]`` (always, when not causal).
    Returns ``out [m, d]``, ``lse [m]`` and optionally the probabilities.
    """
    m, n = q.shape[0], k.shape[0]
    scores = (q @ k.T) * scale                                   # A = Q K^T / sqrt(d_k)
    if causal:
        visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    else:
        visible = np.ones((m, n), dtype=bool)
    masked = np.where(visible, scores, -np.inf)
    row_max = masked.max(axis=1) if n > 0 else np.full(m, -np.inf)
    any_visible = visible.any(axis=1) if n > 0 else np.zeros(m, dtype=bool)
    ref = np.where(any_visible, row_max, 0.0)
    probs = np.where(visible, np.exp(masked - ref[:, None]), 0.0)  # softmax numerator
    denom = probs.sum(axis=1)
    safe = np.where(any_visible, denom, 1.0)
    out = np.where(any_visible[:, None], (probs @ v) / safe[:, None], 0.0)  # O = softmax(A) V
    lse = np.where(any_visible, ref + np.log(safe), -np.inf)
    if return_probs:
        return out, lse, probs / safe[:, None]
    return out, lse


def attend(q, q_offsets, q_pos, seg_offsets, segs, block_table, K_pool, V_pool,
           num_kv_heads, scale=0.0, causal=True, block_size=16, rows=None):
    """MSA over a batch of sequences.

    ``q [total_q, H_q, d]``; sequence ``b`` owns query rows
    ``q_offsets[b]:q_offsets[b+1]`` and segments ``seg_offsets[b]:seg_offsets[b+1]``.
    ``rows`` optionally restricts the computation to a subset of query rows
    (others are returned as NaN).  Returns ``out [total_q, H_q, d]`` and
    ``lse [total_q, H_q]`` in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    total_q, H_q, d = q.shape
    assert H_q % num_kv_heads == 0
    group = H_q // num_kv_heads
    if not scale:
        scale = 1.0 / math.sqrt(d)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    want = np.ones(total_q, dtype=bool)
    if rows is not None:
        want = np.zeros(total_q, dtype=bool)
        want[np.asarray(rows, dtype=np.int64)] = True
    out = np.full((total_q, H_q, d), np.nan)
    lse = np.full((total_q, H_q), np.nan)
    for b in range(len(q_offsets) - 1):
        r = np.arange(q_offsets[b], q_offsets[b + 1])
        r = r[want[r]]
        if len(r) == 0:
            continue
        K, V, k_pos = gather_context(segs[seg_offsets[b]:seg_offsets[b + 1]], block_table,
                                     K_pool, V_pool, block_size)
        for h in range(H_q):
            g = h // group
            o, l = masked_softmax_attention(q[r, h, :], K[:, g, :], V[:, g, :], q_pos[r], k_pos,
                                            scale, causal)
            out[r, h, :] = o
            lse[r, h] = l
    return out, lse


def merge_partials(outs, lses):
    """Combine attention results over disjoint key sets into the result over their union.

    ``outs[i] [..., d]`` is softmax attention over key set i and ``lses[i] [...]``
    its log-sum-exp.  With ``M = max_i lse_i`` and ``w_i = exp(lse_i - M)``:
    ``out = sum_i w_i out_i / sum_i w_i`` and ``lse = M + log(sum_i w_i)``.
    Parts with ``lse = -inf`` (no visible key) get weight 0; if all are empty
    the result is ``out = 0``, ``lse = -inf``.
    """
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])
    M = lses.max(axis=0)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - Ms[None]))
    wsum = w.sum(axis=0)
    safe = np.where(empty, 1.0, wsum)
    out = np.where(empty[..., None], 0.0, (w[..., None] * np.where(w[..., None] > 0, outs, 0.0)).sum(axis=0) / safe[..., None])
    lse = np.where(empty, -np.inf, Ms + np.log(safe))
    return out, lse
