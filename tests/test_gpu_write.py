"""GPU parity of the KV write (msa_write_kv) against the CPU oracle ``oracle.write_kv``.

The write is a copy, so the bar is bit-exact: every slot of the pool after the
GPU write must hold the same bits as the oracle's result on the same seeded
input, including slots the write must leave alone (NaN poison and tails of
partial blocks).  Write-then-attend cases check that msa_forward reads what
the write placed (bf16 bounds of the attention parity tests).
"""
import numpy as np
import pytest
import torch

import kv_cache_attention_msa_amd as msa
import workloads as W
from msa_gpu_util import compare
from oracle import attend, write_kv

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _np_bits(t):
    return _bits(t.contiguous().cpu()).numpy()


def _pool_for(wl, K, V):
    dt = msa.FP32 if wl.dtype == "fp32" else msa.BF16
    return msa.Pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, dt, k=K, v=V)


def _bt(wl):
    bt = torch.from_numpy(wl.block_table.astype(np.int32)).cuda()
    return bt if bt.numel() else torch.zeros(1, dtype=torch.int32, device="cuda")


def _check_whole_pool(wl, fresh, stream=None):
    """GPU write over the dense pool, compared bit for bit with the oracle."""
    print(f"[write] {wl.name} segs={len(fresh.segs)} rows={fresh.rows}", flush=True)
    K, V = wl.dense_pool("cuda")
    K0, V0 = _np_bits(K), _np_bits(V)
    pool = _pool_for(wl, K, V)
    try:
        ks, vs = fresh.k.cuda(), fresh.v.cuda()
        msa.write_kv(pool, ks, vs, fresh.segs, fresh.src_rows, _bt(wl), stream=stream)
        torch.cuda.synchronize()
        Kr, Vr = write_kv(K0, V0, _np_bits(fresh.k), _np_bits(fresh.v), fresh.segs, fresh.src_rows, wl.block_table)
        np.testing.assert_array_equal(_np_bits(K), Kr)
        np.testing.assert_array_equal(_np_bits(V), Vr)
    finally:
        pool.close()


CASES = [
    dict(seed=1, H_q=8, H_kv=2, d=128, dtype="bf16"),
    dict(seed=2, H_q=4, H_kv=4, d=64, dtype="bf16"),
    dict(seed=3, H_q=6, H_kv=3, d=128, dtype="bf16"),   # tasks not a multiple of 4
    dict(seed=4, H_q=2, H_kv=1, d=64, dtype="fp32"),
    dict(seed=5, H_q=8, H_kv=2, d=128, dtype="fp32"),
]


@pytest.mark.parametrize("kw", CASES, ids=lambda k: f"s{k['seed']}_{k['dtype']}_d{k['d']}_kv{k['H_kv']}")
def test_random_cases_bit_exact(kw):
    wl = W.random_case(kw["seed"] + 500, batch=4, H_q=kw["H_q"], H_kv=kw["H_kv"], d=kw["d"], dtype=kw["dtype"],
                       max_ctx=400, max_chunk=90)
    fresh = W.fresh_kv(wl, seed=kw["seed"])
    assert len(fresh.segs) > 0
    _check_whole_pool(wl, fresh)


def test_edge_lengths_bit_exact():
    # lengths 1, 15, 16, 17, 0 and 48 (whole blocks), fresh rows in shuffled order
    wl = W.custom([([(0, 1, 1), (10, 15, 1), (40, 16, 1)], [41]),
                   ([(0, 17, 1), (30, 0, 1), (60, 48, 1), (200, 5, 0)], [100, 101])],
                  H_q=4, H_kv=2, d=128, seed=9, name="edge_lengths")
    fresh = W.fresh_kv(wl, seed=9)
    assert sorted(fresh.segs[:, 1].tolist()) == [0, 1, 15, 16, 17, 48]
    _check_whole_pool(wl, fresh)


def test_nothing_to_write_leaves_pool_alone():
    wl = W.custom([([(0, 40, 0)], [39])], H_q=2, H_kv=1, d=64, seed=3, name="no_fresh")
    fresh = W.fresh_kv(wl, seed=3)
    assert len(fresh.segs) == 0
    K, V = wl.dense_pool("cuda")
    before = _np_bits(K)
    pool = _pool_for(wl, K, V)
    try:
        msa.write_kv(pool, None, None, fresh.segs, fresh.src_rows, _bt(wl))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_np_bits(K), before)
    finally:
        pool.close()


def _oracle_pools_after_write(wl, fresh):
    """fp64 pools (compact over the workload's used blocks) after the oracle write."""
    inv = np.full(wl.num_blocks, -1, dtype=np.int64)
    inv[wl.used_ids] = np.arange(len(wl.used_ids))
    bt_c = inv[wl.block_table]
    Kc = wl.k_blocks.to(torch.float64).numpy()
    Vc = wl.v_blocks.to(torch.float64).numpy()
    Kc, Vc = write_kv(Kc, Vc, fresh.k.to(torch.float64).numpy(), fresh.v.to(torch.float64).numpy(),
                      fresh.segs, fresh.src_rows, np.where(bt_c < 0, 0, bt_c))
    return (W.SparsePool(torch.from_numpy(Kc), wl.used_ids, wl.num_blocks),
            W.SparsePool(torch.from_numpy(Vc), wl.used_ids, wl.num_blocks))


def _write_then_attend(wl, fresh, rows=None, stream=None):
    print(f"[write+attend] {wl.name} rows={'all' if rows is None else len(rows)}", flush=True)
    K, V = wl.dense_pool("cuda")
    pool = _pool_for(wl, K, V)
    try:
        q = wl.q.cuda()
        out = torch.full_like(q, float("nan"))
        lse = torch.full((wl.total_q, wl.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
        bt = _bt(wl)
        ks, vs = fresh.k.cuda(), fresh.v.cuda()
        torch.cuda.synchronize()
        s = stream or torch.cuda.current_stream()
        with torch.cuda.stream(s):
            msa.write_kv(pool, ks, vs, fresh.segs, fresh.src_rows, bt, stream=s)
            msa.forward(q, msa.SegDesc.from_workload(wl), bt, pool, out, lse, stream=s)
        torch.cuda.synchronize()
    finally:
        pool.close()
    Kp, Vp = _oracle_pools_after_write(wl, fresh)
    ref_out, ref_lse = attend(wl.q_f64(), wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, wl.block_table,
                              Kp, Vp, wl.num_kv_heads, scale=wl.scale, causal=bool(wl.causal), rows=rows)
    return compare(wl, out.cpu(), lse.cpu(), ref_out, ref_lse, rows)


def test_write_then_attend_random():
    wl = W.random_case(77, batch=5, H_q=8, H_kv=2, d=128, max_ctx=500, max_chunk=100)
    _write_then_attend(wl, W.fresh_kv(wl, seed=77))


def test_write_then_attend_on_side_stream():
    wl = W.random_case(78, batch=3, H_q=8, H_kv=2, d=128, max_ctx=300, max_chunk=60)
    s = torch.cuda.Stream()
    _write_then_attend(wl, W.fresh_kv(wl, seed=78), stream=s)


# ---- full size: the mixed batch's fresh segments (61 segments, 44 820 rows) ----
@pytest.fixture(scope="module")
def mixed():
    wl = W.config5()
    return wl, W.fresh_kv(wl, seed=5)


def test_mixed_full_size_bit_exact(mixed):
    wl, fresh = mixed
    print(f"[write] {wl.name} full size: {len(fresh.segs)} segments, {fresh.rows} rows", flush=True)
    K, V = wl.dense_pool("cuda")
    K0, V0 = _bits(K).clone(), _bits(V).clone()
    pool = _pool_for(wl, K, V)
    try:
        msa.write_kv(pool, fresh.k.cuda(), fresh.v.cuda(), fresh.segs, fresh.src_rows, _bt(wl))
        torch.cuda.synchronize()
        touched = np.unique(np.concatenate(
            [wl.block_table[s[2]:s[2] + -(-s[1] // 16)] for s in fresh.segs if s[1] > 0]))
        # untouched blocks: identical bits, compared on the device
        mask = torch.ones(wl.num_blocks, dtype=torch.bool, device="cuda")
        mask[torch.from_numpy(touched).cuda()] = False
        assert torch.equal(_bits(K)[mask], K0[mask]) and torch.equal(_bits(V)[mask], V0[mask])
        # touched blocks: the oracle on a compact copy of just those blocks
        inv = np.full(wl.num_blocks, 0, dtype=np.int64)
        inv[touched] = np.arange(len(touched))
        idx = torch.from_numpy(touched).cuda()
        Kr, Vr = write_kv(K0[idx].cpu().numpy(), V0[idx].cpu().numpy(), _np_bits(fresh.k), _np_bits(fresh.v),
                          fresh.segs, fresh.src_rows, inv[wl.block_table])
        np.testing.assert_array_equal(_bits(K)[idx].cpu().numpy(), Kr)
        np.testing.assert_array_equal(_bits(V)[idx].cpu().numpy(), Vr)
    finally:
        pool.close()


def test_mixed_full_size_write_then_attend(mixed):
    wl, fresh = mixed
    rng = np.random.default_rng(55)
    rows = np.unique(np.concatenate([rng.choice(wl.total_q, 48, replace=False),
                                     wl.q_offsets[1:] - 1]))
    _write_then_attend(wl, fresh, rows=rows)


def test_write_block_id_check_option():
    """MSA_OPT_CHECK_BLOCK_IDS on msa_write_kv: an out-of-range destination id
    fails the call before the write kernel, and the pool is left unchanged."""
    wl = W.random_case(505, batch=2, H_q=8, H_kv=2, d=128, max_ctx=300, max_chunk=60)
    fresh = W.fresh_kv(wl, seed=505)
    K, V = wl.dense_pool("cuda")
    K0, V0 = _np_bits(K), _np_bits(V)
    pool = _pool_for(wl, K, V)
    try:
        pool.set_option(msa.OPT_CHECK_BLOCK_IDS, 1)
        bt = _bt(wl)
        dst = int(fresh.segs[0, 2])
        bt[dst] = wl.num_blocks + 3
        with pytest.raises(msa.MsaError) as ei:
            msa.write_kv(pool, fresh.k.cuda(), fresh.v.cuda(), fresh.segs, fresh.src_rows, bt)
        torch.cuda.synchronize()
        assert ei.value.code == msa.ERR_INVALID_ARG and "block_table[" in str(ei.value)
        np.testing.assert_array_equal(_np_bits(K), K0)
        np.testing.assert_array_equal(_np_bits(V), V0)
    finally:
        pool.close()
