"""Pins for the KV write (recompute-scatter) oracle, ``oracle.write_kv``.

The write is a pure placement, so it is pinned by literal slot contents of a
hand example, by the attention oracle's independently pinned gather (a round
trip), by untouched slots, and by write-then-attend against torch's fp64
causal attention over the unpaged rows.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attend, gather_context, write_kv

BS = 16


def _nan_pool(num_blocks, H, d, dtype=np.float64):
    return np.full((num_blocks, H, BS, d), np.nan, dtype=dtype)


def _rows(n, H, d, base):
    r = np.arange(n)[:, None, None] * 100 + np.arange(H)[None, :, None] * 10 + np.arange(d)[None, None, :]
    return (r + base).astype(np.float64)


def test_hand_example_literal_slots():
    # block_table [4, 1, 5, 0, 3]; segment A: 18 tokens from bt index 1, fresh
    # rows 2..19; segment B: 3 tokens from bt index 4, fresh rows 0..2.
    K0, V0 = _nan_pool(6, 2, 3), _nan_pool(6, 2, 3)
    ks, vs = _rows(20, 2, 3, 0), _rows(20, 2, 3, 50000)
    segs = [(100, 18, 1, 1), (400, 3, 4, 1)]
    K, V = write_kv(K0, V0, ks, vs, segs, [2, 0], [4, 1, 5, 0, 3])
    assert K[1, 0, 0].tolist() == [200, 201, 202]          # A token 0 -> block 1 slot 0, row 2
    assert K[1, 1, 15].tolist() == [1710, 1711, 1712]      # A token 15 -> block 1 slot 15, row 17, head 1
    assert K[5, 0, 0].tolist() == [1800, 1801, 1802]       # A token 16 -> block 5 slot 0, row 18
    assert K[5, 1, 1].tolist() == [1910, 1911, 1912]       # A token 17 -> block 5 slot 1, row 19
    assert np.isnan(K[5, :, 2:]).all()                     # tail of A's last block untouched
    assert K[3, 0, 0].tolist() == [0, 1, 2]                # B token 0 -> block 3 slot 0, row 0
    assert K[3, 1, 2].tolist() == [210, 211, 212]          # B token 2 -> block 3 slot 2, row 2, head 1
    assert np.isnan(K[3, :, 3:]).all()
    assert np.isnan(K[0]).all() and np.isnan(K[2]).all() and np.isnan(K[4]).all()
    assert V[1, 0, 0].tolist() == [50200, 50201, 50202]
    assert V[3, 1, 2].tolist() == [50210, 50211, 50212]
    assert int((~np.isnan(K[..., 0])).sum()) == (18 + 3) * 2
    assert np.isnan(K0).all()                              # inputs are not modified


def _random_layout(rng, n_segs, num_blocks, max_len=70):
    lens = rng.integers(1, max_len, size=n_segs)
    nblk = -(-lens // BS)
    ids = rng.permutation(num_blocks)[: int(nblk.sum())]
    bt = rng.permutation(ids)
    segs, bt_start, pos = [], 0, 0
    for L, nb in zip(lens, nblk):
        segs.append((pos, int(L), bt_start, 1))
        bt_start += int(nb)
        pos += int(L) + int(rng.integers(0, 40))
    src_order = rng.permutation(n_segs)
    src_rows = np.zeros(n_segs, dtype=np.int64)
    row = 0
    for s in src_order:
        src_rows[s] = row
        row += int(lens[s])
    return segs, src_rows, bt, row


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_through_attention_gather(seed):
    rng = np.random.default_rng(seed)
    H, d, nb = 3, 8, 64
    segs, src_rows, bt, n_rows = _random_layout(rng, 5, nb)
    ks, vs = rng.standard_normal((n_rows, H, d)), rng.standard_normal((n_rows, H, d))
    K, V = write_kv(_nan_pool(nb, H, d), _nan_pool(nb, H, d), ks, vs, segs, src_rows, bt)
    Kg, Vg, pos = gather_context(segs, bt, K, V)
    want = np.concatenate([np.arange(r, r + s[1]) for s, r in zip(segs, src_rows)])
    np.testing.assert_array_equal(Kg, ks[want])
    np.testing.assert_array_equal(Vg, vs[want])


def test_untouched_slots_keep_their_bits():
    rng = np.random.default_rng(7)
    H, d, nb = 2, 4, 40
    segs, src_rows, bt, n_rows = _random_layout(rng, 4, nb)
    K0 = rng.integers(0, 1 << 16, size=(nb, H, BS, d)).astype(np.uint16)   # raw bf16 bit patterns
    V0 = rng.integers(0, 1 << 16, size=(nb, H, BS, d)).astype(np.uint16)
    ks = rng.integers(0, 1 << 16, size=(n_rows, H, d)).astype(np.uint16)
    vs = rng.integers(0, 1 << 16, size=(n_rows, H, d)).astype(np.uint16)
    K, V = write_kv(K0, V0, ks, vs, segs, src_rows, bt)
    covered = np.zeros((nb, BS), dtype=bool)
    for s in segs:
        for i in range(s[1]):
            covered[bt[s[2] + i // BS], i % BS] = True
    assert covered.sum() == sum(s[1] for s in segs)
    np.testing.assert_array_equal(K.transpose(0, 2, 1, 3)[~covered], K0.transpose(0, 2, 1, 3)[~covered])
    np.testing.assert_array_equal(V.transpose(0, 2, 1, 3)[~covered], V0.transpose(0, 2, 1, 3)[~covered])
    assert K.dtype == np.uint16


def test_segment_order_does_not_matter():
    rng = np.random.default_rng(11)
    H, d, nb = 2, 4, 48
    segs, src_rows, bt, n_rows = _random_layout(rng, 6, nb)
    ks, vs = rng.standard_normal((n_rows, H, d)), rng.standard_normal((n_rows, H, d))
    K1, V1 = write_kv(_nan_pool(nb, H, d), _nan_pool(nb, H, d), ks, vs, segs, src_rows, bt)
    perm = rng.permutation(len(segs))
    K2, V2 = write_kv(_nan_pool(nb, H, d), _nan_pool(nb, H, d), ks, vs, [segs[i] for i in perm],
                      src_rows[perm], bt)
    np.testing.assert_array_equal(K1, K2)
    np.testing.assert_array_equal(V1, V2)


def test_write_then_attend_equals_causal_attention():
    # A 75-token sequence computed fresh, written as three segments into
    # scattered blocks, then attended by all 75 rows: plain causal attention.
    rng = np.random.default_rng(3)
    N, H, d, nb = 75, 2, 16, 20
    k, v, q = (rng.standard_normal((N, H, d)) for _ in range(3))
    cuts = [0, 23, 48, N]
    bt = rng.permutation(nb)[:8]
    segs, src_rows, bt_start = [], [], 0
    for a, b in zip(cuts[:-1], cuts[1:]):
        segs.append((a, b - a, bt_start, 1))
        src_rows.append(a)
        bt_start += -(-(b - a) // BS)
    K, V = write_kv(_nan_pool(nb, H, d), _nan_pool(nb, H, d), k, v, segs, src_rows, bt)
    out, lse = attend(q, [0, N], np.arange(N), [0, len(segs)], np.array(segs), bt, K, V, H)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2))) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(out, ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
