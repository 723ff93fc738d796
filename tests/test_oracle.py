"""Pins for the fp64 oracle: each test checks it against something other than itself.

Brute force (scalar loops, no max subtraction), torch's fp64 scaled-dot-product
attention, hand-worked examples, closed forms, invariants and the log-sum-exp
merge identity.  Each one is chosen so that a plausible slip in the oracle (a
flipped mask, a wrong GQA index, a dropped scale, position taken from gather
order, a wrong log base) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attend, gather_context, masked_softmax_attention, merge_partials

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def run_oracle(wl, rows=None, scale=None):
    K, V = wl.dense_pool()
    K = K.to(torch.float64).numpy()
    V = V.to(torch.float64).numpy()
    return attend(wl.q_f64(), wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, wl.block_table,
                  K, V, wl.num_kv_heads, scale=wl.scale if scale is None else scale,
                  causal=bool(wl.causal), rows=rows)


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------
def brute_force(wl):
    """Scalar loops straight from the definition: walk each segment token by
    token through the block table, sum exp(score) without any max shift."""
    K, V = wl.dense_pool()
    K = K.to(torch.float64).numpy()
    V = V.to(torch.float64).numpy()
    q = wl.q_f64()
    Hq, Hkv, d = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    scale = wl.scale or 1.0 / math.sqrt(d)
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    for b in range(wl.batch):
        keys = []
        for (p0, ln, bt0, _f) in wl.seg_list(b):
            for i in range(ln):
                blk = int(wl.block_table[bt0 + i // 16])
                keys.append((p0 + i, blk, i % 16))
        for r in range(wl.q_offsets[b], wl.q_offsets[b + 1]):
            for h in range(Hq):
                kvh = h * Hkv // Hq
                tot = 0.0
                acc = [0.0] * d
                for (kp, blk, slot) in keys:
                    if wl.causal and kp > wl.q_pos[r]:
                        continue
                    s = 0.0
                    for c in range(d):
                        s += q[r, h, c] * K[blk, kvh, slot, c]
                    e = math.exp(s * scale)
                    tot += e
                    for c in range(d):
                        acc[c] += e * V[blk, kvh, slot, c]
                if tot == 0.0:
                    out[r, h] = 0.0
                    lse[r, h] = -math.inf
                else:
                    out[r, h] = [a / tot for a in acc]
                    lse[r, h] = math.log(tot)
    return out, lse


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    specs = []
    for _ in range(2):
        n = int(rng.integers(1, 4))
        segs, pos = [], int(rng.integers(0, 5))
        for _ in range(n):
            ln = int(rng.integers(1, 14))
            segs.append((pos, ln))
            pos += ln + int(rng.integers(0, 3))
        qp = sorted(rng.choice(np.arange(-2, pos + 2), size=int(rng.integers(1, 5)), replace=False).tolist())
        specs.append((segs, qp))
    wl = W.custom(specs, H_q=4, H_kv=2, d=8, dtype="fp32", seed=seed, qscale=1.0, kvscale=1.0)
    o, l = run_oracle(wl)
    bo, bl = brute_force(wl)
    assert np.allclose(o, bo, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(l), np.isneginf(bl))
    fin = np.isfinite(bl)
    assert np.allclose(l[fin], bl[fin], rtol=0, atol=1e-12)


def test_brute_force_noncausal_and_scale():
    specs = [([(0, 5), (9, 7)], [3, 12]), ([(2, 17)], [0])]
    wl = W.custom(specs, H_q=2, H_kv=1, d=4, dtype="fp32", seed=7, qscale=1.0, kvscale=1.0,
                  scale=0.37, causal=0)
    o, l = run_oracle(wl)
    bo, bl = brute_force(wl)
    assert np.allclose(o, bo, atol=1e-12) and np.allclose(l, bl, atol=1e-12)


def test_brute_force_config1():
    wl = W.config1()
    o, l = run_oracle(wl)
    bo, bl = brute_force(wl)
    assert np.allclose(o, bo, atol=1e-12) and np.allclose(l, bl, atol=1e-12)


# ---------------------------------------------------------------------------
# hand-worked examples (tests/golden)
# ---------------------------------------------------------------------------
def _golden_case(ex):
    d = 2
    n_blocks = 2 * len(ex["segments"]) + 2
    K = np.full((n_blocks, 1, 16, d), np.nan)
    V = np.full((n_blocks, 1, 16, d), np.nan)
    segs, bt = [], []
    free = list(range(n_blocks - 1, -1, -1))
    for (p0, ln), ws, vs in zip(ex["segments"], ex["segment_weights"], ex["segment_values"]):
        blk = free.pop(0)  # one block per segment (all segments are short)
        segs.append((p0, ln, len(bt), 0))
        bt.append(blk)
        for i in range(ln):
            K[blk, 0, i] = [math.log(ws[i]), 0.0]
            V[blk, 0, i] = vs[i]
    q = np.array([[qq["q"]] for qq in ex["queries"]], dtype=np.float64)
    q_pos = np.array([qq["pos"] for qq in ex["queries"]])
    return q, q_pos, np.array(segs), np.array(bt), K, V


def test_golden_hand_examples():
    with open(GOLDEN) as f:
        data = json.load(f)
    for ex in data["examples"]:
        q, q_pos, segs, bt, K, V = _golden_case(ex)
        o, l = attend(q, [0, len(q)], q_pos, [0, len(segs)], segs, bt, K, V, 1, scale=1.0)
        exp_o = np.array([[float(Fraction(x)) for x in row] for row in ex["expected_out_fraction"]])
        exp_l = np.log(np.array(ex["expected_lse_of"], dtype=np.float64))
        assert np.allclose(o[:, 0, :], exp_o, atol=1e-13), ex["name"]
        assert np.allclose(l[:, 0], exp_l, atol=1e-13), ex["name"]


# ---------------------------------------------------------------------------
# textbook special case: torch fp64 scaled-dot-product attention
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_single_segment_equals_causal_sdpa(Hq, Hkv):
    N, d = 45, 16
    wl = W.custom([([(0, N)], list(range(N)))], H_q=Hq, H_kv=Hkv, d=d, dtype="fp32", seed=3,
                  qscale=1.0, kvscale=1.0)
    o, l = run_oracle(wl)
    Kc, Vc, kp = gather_context(wl.segs, wl.block_table, *[x.to(torch.float64).numpy() for x in wl.dense_pool()])
    assert np.array_equal(kp, np.arange(N))
    q = torch.from_numpy(wl.q_f64()).permute(1, 0, 2).unsqueeze(0)          # [1, Hq, N, d]
    k = torch.from_numpy(Kc).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0).unsqueeze(0)
    v = torch.from_numpy(Vc).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0).unsqueeze(0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_chunk_after_context_equals_bottom_right_sdpa():
    ctx, c, d, H = 37, 11, 16, 2
    wl = W.custom([([(0, ctx), (ctx, c)], list(range(ctx, ctx + c)))], H_q=H, H_kv=H, d=d,
                  dtype="fp32", seed=4, qscale=1.0, kvscale=1.0)
    o, _ = run_oracle(wl)
    pools = [x.to(torch.float64).numpy() for x in wl.dense_pool()]
    Kc, Vc, kp = gather_context(wl.seg_list(0), wl.block_table, *pools)
    order = np.argsort(kp)
    Kc, Vc = Kc[order], Vc[order]
    q = torch.from_numpy(wl.q_f64()).permute(1, 0, 2).unsqueeze(0)
    k = torch.from_numpy(Kc).permute(1, 0, 2).unsqueeze(0)
    v = torch.from_numpy(Vc).permute(1, 0, 2).unsqueeze(0)
    mask = torch.ones(c, ctx + c, dtype=torch.bool).tril(diagonal=ctx)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    assert np.allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def _with_segs(wl, segs, seg_offsets=None, block_table=None, q_pos=None):
    import copy
    w2 = copy.copy(wl)
    w2.segs = np.asarray(segs, dtype=np.int32).reshape(-1, 4)
    if seg_offsets is not None:
        w2.seg_offsets = np.asarray(seg_offsets, dtype=np.int32)
    if block_table is not None:
        w2.block_table = np.asarray(block_table, dtype=np.int32)
    if q_pos is not None:
        w2.q_pos = np.asarray(q_pos, dtype=np.int32)
    return w2


def test_reorder_segments_invariant():
    wl = W.random_case(11, batch=3, d=32)
    o, l = run_oracle(wl)
    rng = np.random.default_rng(0)
    segs = []
    for b in range(wl.batch):
        s = wl.segs[wl.seg_offsets[b]:wl.seg_offsets[b + 1]]
        segs.extend(s[rng.permutation(len(s))])
    o2, l2 = run_oracle(_with_segs(wl, segs))
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(l, l2, atol=1e-12)


def test_split_segment_invariant():
    """Split a segment: its tail becomes a new descriptor whose blocks are copies
    placed elsewhere in the pool."""
    wl = W.custom([([(0, 70), (80, 20)], [95, 99, 100])], H_q=4, H_kv=1, d=16, dtype="fp32",
                  seed=5, num_blocks=20, qscale=1.0, kvscale=1.0)
    o, l = run_oracle(wl)
    K, V = [x.to(torch.float64).numpy() for x in wl.dense_pool()]
    seg = [s for s in wl.seg_list(0) if s[1] == 70][0]
    other = [s for s in wl.seg_list(0) if s[1] != 70]
    p0, ln, bt0, f = seg
    used = set(int(x) for x in wl.block_table)
    free = [i for i in range(wl.num_blocks) if i not in used]
    bt = list(wl.block_table)
    head = (p0, 32, bt0, f)
    tail_start = len(bt)
    for j in range(2, 5):                      # blocks 2..4 of the segment hold tokens 32..69
        dst = free.pop()
        K[dst] = K[bt[bt0 + j]]
        V[dst] = V[bt[bt0 + j]]
        K[bt[bt0 + j]] = np.nan                 # the old copy is no longer referenced
        V[bt[bt0 + j]] = np.nan
        bt.append(dst)
    tail = (p0 + 32, ln - 32, tail_start, f)
    segs = [tail, other[0], head]
    o2, l2 = attend(wl.q_f64(), wl.q_offsets, wl.q_pos, [0, 3], np.array(segs), np.array(bt), K, V,
                    wl.num_kv_heads)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(l, l2, atol=1e-12)


def test_position_shift_and_gap_invariant():
    wl = W.random_case(12, batch=2, d=16, gaps=False)
    o, l = run_oracle(wl)
    shift = _with_segs(wl, wl.segs + np.array([1000, 0, 0, 0]), q_pos=wl.q_pos + 1000)
    o2, l2 = run_oracle(shift)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(l, l2, atol=1e-12)
    # order-preserving gaps: every position p maps to p + 3 * (number of segments starting at <= p)
    segs = wl.segs.copy()
    qp = wl.q_pos.astype(np.int64).copy()
    for b in range(wl.batch):
        s0, s1 = wl.seg_offsets[b], wl.seg_offsets[b + 1]
        starts = np.sort(wl.segs[s0:s1, 0])
        for i in range(s0, s1):
            segs[i, 0] += 3 * np.searchsorted(starts, wl.segs[i, 0], side="right")
        for r in range(wl.q_offsets[b], wl.q_offsets[b + 1]):
            qp[r] += 3 * np.searchsorted(starts, wl.q_pos[r], side="right")
    o3, l3 = run_oracle(_with_segs(wl, segs, q_pos=qp))
    assert np.allclose(o, o3, atol=1e-12) and np.allclose(l, l3, atol=1e-12)


def test_poison_outside_segments_has_no_effect():
    wl = W.random_case(13, batch=2, d=16)
    K, V = [x.to(torch.float64).numpy() for x in wl.dense_pool()]
    assert np.isnan(K).any()
    o, l = attend(wl.q_f64(), wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, wl.block_table, K, V,
                  wl.num_kv_heads)
    assert np.isfinite(o).all()
    K2 = np.where(np.isnan(K), 1e30, K)
    V2 = np.where(np.isnan(V), -1e30, V)
    o2, l2 = attend(wl.q_f64(), wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, wl.block_table, K2, V2,
                    wl.num_kv_heads)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_probabilities_sum_to_one_and_respect_mask():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((9, 8)) * 3
    k = rng.standard_normal((30, 8))
    v = rng.standard_normal((30, 8))
    kp = rng.permutation(40)[:30]
    qp = np.array([-1, 0, 5, 10, 20, 30, 39, 50, 2])
    _, _, p = masked_softmax_attention(q, k, v, qp, kp, 0.3, True, return_probs=True)
    sums = p.sum(axis=1)
    has = (kp[None, :] <= qp[:, None]).any(axis=1)
    assert np.allclose(sums[has], 1.0, atol=1e-12) and np.all(sums[~has] == 0)
    assert np.all(p[kp[None, :] > qp[:, None]] == 0)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_zero_query_gives_mean_of_visible_values():
    wl = W.random_case(14, batch=3, d=16)
    wl.q = torch.zeros_like(wl.q)
    o, l = run_oracle(wl)
    K, V = [x.to(torch.float64).numpy() for x in wl.dense_pool()]
    for b in range(wl.batch):
        _, Vc, kp = gather_context(wl.seg_list(b), wl.block_table, K, V)
        for r in range(wl.q_offsets[b], wl.q_offsets[b + 1]):
            vis = kp <= wl.q_pos[r]
            for h in range(wl.num_q_heads):
                g = h // (wl.num_q_heads // wl.num_kv_heads)
                if vis.sum() == 0:
                    assert np.all(o[r, h] == 0) and np.isneginf(l[r, h])
                else:
                    assert np.allclose(o[r, h], Vc[vis, g].mean(axis=0), atol=1e-12)
                    assert abs(l[r, h] - math.log(vis.sum())) < 1e-12


def test_single_visible_key_closed_form():
    wl = W.custom([([(10, 5), (0, 3)], [0, 10])], H_q=2, H_kv=1, d=8, dtype="fp32", seed=9,
                  qscale=1.0, kvscale=1.0)
    o, l = run_oracle(wl)
    K, V = [x.to(torch.float64).numpy() for x in wl.dense_pool()]
    Kc, Vc, kp = gather_context(wl.seg_list(0), wl.block_table, K, V)
    j = int(np.where(kp == 0)[0][0])
    q = wl.q_f64()
    for h in range(2):
        assert np.allclose(o[0, h], Vc[j, 0], atol=1e-14)
        assert abs(l[0, h] - q[0, h] @ Kc[j, 0] / math.sqrt(8)) < 1e-13


def test_constant_values_and_gqa_head_probe():
    wl = W.random_case(15, batch=2, H_q=8, H_kv=4, d=16, dtype="fp32")
    # V of kv head g is the constant g + 1: output of q head h must be h // 2 + 1
    wl.v_blocks = torch.zeros_like(wl.v_blocks) + torch.arange(1, 5, dtype=torch.float32).view(1, 4, 1, 1)
    o, l = run_oracle(wl)
    has = np.isfinite(l)
    for h in range(8):
        assert np.allclose(o[has[:, h], h], h // 2 + 1, atol=1e-12)


def test_peaky_scores_follow_hard_max():
    """Very large scores: the output must equal the value of the top key
    (softmax -> one-hot), finite, with lse equal to the top score."""
    wl = W.custom([([(0, 40), (50, 30)], [45, 79, 90])], H_q=2, H_kv=1, d=16, dtype="fp32", seed=21,
                  qscale=1.0, kvscale=1.0)
    wl.q = wl.q * 2000.0
    o, l = run_oracle(wl)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    K, V = [x.to(torch.float64).numpy() for x in wl.dense_pool()]
    Kc, Vc, kp = gather_context(wl.seg_list(0), wl.block_table, K, V)
    q = wl.q_f64()
    for r in range(3):
        for h in range(2):
            s = (Kc[:, 0] @ q[r, h]) / 4.0
            s[kp > wl.q_pos[r]] = -np.inf
            top2 = np.sort(s)[-2:]
            assert top2[1] - top2[0] > 40
            j = int(np.argmax(s))
            assert np.allclose(o[r, h], Vc[j, 0], atol=1e-12)
            assert abs(l[r, h] - s[j]) < 1e-9


# ---------------------------------------------------------------------------
# log-sum-exp merge of partial results
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [16, 17])
def test_lse_merge_identity(seed):
    wl = W.random_case(seed, batch=3, d=16)
    o, l = run_oracle(wl)
    rng = np.random.default_rng(seed)
    parts = [[], [], []]
    offs = [[0], [0], [0]]
    for b in range(wl.batch):
        s = wl.segs[wl.seg_offsets[b]:wl.seg_offsets[b + 1]]
        which = rng.integers(0, 3, size=len(s))
        for p in range(3):
            parts[p].extend(s[which == p])
            offs[p].append(len(parts[p]))
    res = [run_oracle(_with_segs(wl, parts[p] if parts[p] else np.zeros((0, 4)), seg_offsets=offs[p]))
           for p in range(3)]
    mo, ml = merge_partials([r[0] for r in res], [r[1] for r in res])
    assert np.allclose(mo, o, atol=1e-12)
    fin = np.isfinite(l)
    assert np.array_equal(fin, np.isfinite(ml)) and np.allclose(ml[fin], l[fin], atol=1e-12)


def test_row_subset_matches_full():
    wl = W.random_case(18, batch=3, d=16)
    o, l = run_oracle(wl)
    rows = [0, 3, wl.total_q - 1]
    o2, l2 = run_oracle(wl, rows=rows)
    assert np.array_equal(o[rows], o2[rows]) and np.array_equal(l[rows], l2[rows])
    others = np.setdiff1d(np.arange(wl.total_q), rows)
    assert np.isnan(o2[others]).all()
