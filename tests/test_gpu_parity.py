"""GPU parity: libmsa (HIP, gfx950) against the fp64 oracle on the same seeded inputs.

Bounds: fp32 inputs max-abs 1e-5; bf16 inputs max-abs 2e-2 and mean-abs 2e-3,
applied to out and to lse.  Pools hold NaN in every slot outside the
segments, so a read outside them shows up as a non-finite output.
"""
import sys

import numpy as np
import pytest
import torch

import kv_cache_attention_msa_amd as msa
import workloads as W
from msa_gpu_util import GpuCase, compare, oracle_result

pytestmark = pytest.mark.gpu


def _check(wl, split_blocks=0, rows=None, chunk_waves=0):
    print(f"[parity] {wl.name} split_blocks={split_blocks} chunk_waves={chunk_waves}", flush=True)
    case = GpuCase(wl)
    try:
        out, lse = case.run(split_blocks, chunk_waves=chunk_waves)
    finally:
        case.close()
    ref_out, ref_lse = oracle_result(wl, rows)
    return compare(wl, out, lse, ref_out, ref_lse, rows)


# ---- configuration 1 (fp32) ------------------------------------------------
def test_config1_fp32():
    _check(W.config1())


def test_config1_fp32_split_and_merge():
    _check(W.config1(), split_blocks=1)


# ---- small bf16 cases ---------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_random_bf16(seed):
    H = [(8, 2), (32, 8), (4, 4), (64, 8), (16, 1), (6, 2)][seed]
    d = 64 if seed % 2 else 128
    _check(W.random_case(seed, batch=4, H_q=H[0], H_kv=H[1], d=d))


@pytest.mark.parametrize("seed", range(3))
def test_random_bf16_forced_split(seed):
    _check(W.random_case(20 + seed, batch=3, H_q=8, H_kv=2, d=128, max_ctx=600), split_blocks=3)


@pytest.mark.parametrize("seed", range(4))
def test_random_bf16_eight_wave_chunk(seed):
    """The chunk launch forced to 8-wave work-groups (256-row tiles) on small
    mixed batches: the decode items then run on half of each work-group while
    the other waves only join its barriers.  (By itself the planner takes 8
    waves only for long-context prefill-only batches, e.g. the heavy-
    fragmentation workload of the full-size test.)"""
    H = [(8, 2), (32, 8), (64, 8), (6, 2)][seed]
    d = 128 if seed % 2 == 0 else 64
    wl = W.random_case(60 + seed, batch=4, H_q=H[0], H_kv=H[1], d=d, max_ctx=700, max_chunk=300)
    _check(wl, chunk_waves=8)
    _check(wl, split_blocks=3, chunk_waves=8)
    _check(wl, chunk_waves=4)


def test_random_sweep():
    """40 seeded small batches over the parameter space at once: GQA ratio,
    head_dim, batch size, context and chunk lengths, decode share, forced KV
    splits and the chunk work-group size, each against the oracle."""
    rng = np.random.default_rng(2024)
    groups = [(1, 1), (2, 1), (4, 1), (8, 2), (16, 2), (12, 4), (32, 8), (64, 8), (128, 1)]
    for i in range(40):
        hq, hkv = groups[int(rng.integers(len(groups)))]
        d = int(rng.choice([64, 128]))
        wl = W.random_case(300 + i, batch=int(rng.integers(1, 7)), H_q=hq, H_kv=hkv, d=d,
                           max_ctx=int(rng.integers(16, 900)), max_chunk=int(rng.integers(1, 260)),
                           decode_frac=float(rng.choice([0.0, 0.3, 0.7, 1.0])), qscale=float(rng.choice([0.5, 2.0])))
        _check(wl, split_blocks=int(rng.choice([0, 0, 1, 3, 7])), chunk_waves=int(rng.choice([0, 4, 8])))


def test_random_fp32_cases():
    for seed in range(3):
        _check(W.random_case(40 + seed, batch=3, H_q=4, H_kv=2, d=64, dtype="fp32"))
        _check(W.random_case(50 + seed, batch=2, H_q=2, H_kv=1, d=128, dtype="fp32"), split_blocks=2)
    # a GQA group (32) larger than the fp32 tile's 16 waves: each wave takes several rows
    _check(W.random_case(55, batch=2, H_q=32, H_kv=1, d=64, dtype="fp32"))


def test_asymcache_layout():
    """Eq. 5 layout: cached l1 | recomputed q1 (with queries) | cached suffix l2 | new q2 (with queries).
    Rows of q1 must not see l2."""
    l1, q1, l2, q2 = 300, 70, 200, 90
    segs = [(0, l1), (l1, q1, W.SEG_FRESH), (l1 + q1, l2), (l1 + q1 + l2, q2, W.SEG_FRESH)]
    qp = list(range(l1, l1 + q1)) + list(range(l1 + q1 + l2, l1 + q1 + l2 + q2))
    for d in (64, 128):
        _check(W.custom([(segs, qp)], H_q=32, H_kv=8, d=d, seed=5))


def test_edge_cases():
    cases = [
        # length-1 segments, lengths not multiple of 16, a query before all keys
        W.custom([([(5, 1), (7, 1), (20, 17), (50, 33)], [0, 6, 7, 30, 82])], H_q=8, H_kv=2, d=128, seed=1),
        # sequence with no segments, sequence with no queries, decode token
        W.custom([([], [3, 4]), ([(0, 40)], []), ([(0, 100), (200, 5)], [204])], H_q=8, H_kv=2, d=128, seed=2),
        # MHA (H_q == H_kv) and d = 64
        W.custom([([(0, 130), (140, 50)], list(range(140, 190)))], H_q=4, H_kv=4, d=64, seed=3),
        # non-causal
        W.custom([([(0, 70), (100, 30)], [10, 50, 120])], H_q=8, H_kv=2, d=128, seed=4, causal=0),
        # peaky scores (q x 8) stress max subtraction and rescaling
        W.custom([([(0, 400), (500, 100)], list(range(500, 600)))], H_q=8, H_kv=2, d=128, seed=6, qscale=4.0),
        # decode with several query tokens per sequence and GQA 8
        W.custom([([(0, 1000)], [997, 998, 999])], H_q=16, H_kv=2, d=128, seed=7),
        # explicit scale
        W.custom([([(0, 77)], list(range(60, 77)))], H_q=4, H_kv=1, d=128, seed=8, scale=0.05),
        # largest GQA ratio (128 q heads on one kv head: one token per 128-row chunk tile), and a
        # decode token whose group (16) exceeds the decode kernel's 8 rows
        W.custom([([(0, 90), (100, 40)], [139, 120, 95])], H_q=128, H_kv=1, d=64, seed=9),
        W.custom([([(0, 500)], [499]), ([(0, 33)], [32])], H_q=32, H_kv=2, d=128, seed=10),
    ]
    for wl in cases:
        _check(wl)
        _check(wl, split_blocks=2)


@pytest.mark.parametrize("factor", [30.0, 300.0])
def test_reference_moves_mid_row(factor):
    """Scores that jump by far more than 2^20 (log2 domain) partway through a
    row: the kernel's per-row reference must move and rescale mid-row, both
    within a step and across KV splits."""
    wl = W.custom([([(0, 300), (300, 100), (400, 200, W.SEG_FRESH)], list(range(400, 600)))],
                  H_q=8, H_kv=2, d=128, seed=12)
    first, second = -(-300 // 16), -(-100 // 16)          # blocks of the first two segments, in build order
    k = wl.k_blocks.float()
    k[first:first + second] *= factor                     # the middle segment's keys dominate
    wl.k_blocks = k.to(torch.bfloat16)
    _check(wl)
    _check(wl, split_blocks=3)


def test_timing_records_every_launch():
    """With timing on, every launch of a kind is recorded once, with a positive duration."""
    wl = W.random_case(70, batch=3, H_q=8, H_kv=2, d=128, max_ctx=600, max_chunk=80)
    case = GpuCase(wl)
    try:
        case.pool.set_option(msa.OPT_TIMING, 1)
        case.pool.set_option(msa.OPT_SPLIT_BLOCKS, 3)     # forces split items and the merge kernel
        for k in range(5):
            case.pool.kernel_time(k, reset=True)
        for _ in range(3):
            msa.forward(case.q, case.desc, case.bt, case.pool, case.out, case.lse)
        torch.cuda.synchronize()
        for kind in (msa.KERNEL_UPLOAD, msa.KERNEL_MERGE):
            total, n = case.pool.kernel_time(kind)
            samples = case.pool.kernel_samples(kind)
            assert n == 3 and len(samples) == 3, (kind, n, len(samples))
            assert (samples > 0).all() and abs(samples.sum() - total) < 1e-3 * max(total, 1e-3)
        launched = sum(case.pool.kernel_time(k)[1] for k in (msa.KERNEL_PREFILL, msa.KERNEL_DECODE))
        assert launched >= 3
        case.pool.kernel_time(msa.KERNEL_UPLOAD, reset=True)
        assert len(case.pool.kernel_samples(msa.KERNEL_UPLOAD)) == 0
    finally:
        case.close()


def test_empty_batch_and_no_queries():
    wl = W.custom([([(0, 40)], [])], H_q=4, H_kv=1, d=128)
    case = GpuCase(wl)
    try:
        msa.forward(case.q, case.desc, case.bt, case.pool, case.out, case.lse)
        torch.cuda.synchronize()
    finally:
        case.close()


def test_deterministic():
    wl = W.random_case(60, batch=3, H_q=32, H_kv=8, d=128, max_ctx=900)
    case = GpuCase(wl)
    try:
        ref = case.run(split_blocks=5)
        for _ in range(4):
            o, l = case.run(split_blocks=5)
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                               ref[0].view(torch.int16) if o.dtype == torch.bfloat16 else ref[0])
            assert torch.equal(l, ref[1]) or torch.equal(torch.isnan(l), torch.isnan(ref[1]))
    finally:
        case.close()


def test_back_to_back_calls_with_changing_plans():
    # Consecutive calls pack their plans into a ring of pinned staging
    # buffers, each copied by a kernel on the caller's stream into the pool's
    # one device plan buffer ahead of that call's attention kernels; calls are
    # queued without a host sync in between and their plans differ in size
    # (staging and plan buffers grow on the way).
    wl = W.random_case(62, batch=4, H_q=32, H_kv=8, d=128, max_ctx=700)
    case = GpuCase(wl)
    splits = [0, 3, 1, 7, 0, 2, 1]
    outs = []
    try:
        for sb in splits:
            case.pool.set_option(msa.OPT_SPLIT_BLOCKS, sb)
            o = torch.full_like(case.q, float("nan"))
            l = torch.full((wl.total_q, wl.num_q_heads), float("nan"), device="cuda")
            msa.forward(case.q, case.desc, case.bt, case.pool, o, l)
            outs.append((o, l))
        torch.cuda.synchronize()
    finally:
        case.close()
    ref_out, ref_lse = oracle_result(wl)
    for sb, (o, l) in zip(splits, outs):
        print(f"[parity] back-to-back split_blocks={sb}", flush=True)
        compare(wl, o.cpu(), l.cpu(), ref_out, ref_lse)


def test_block_table_written_on_the_stream_between_calls():
    # The kernels read pool block ids through the block table on the call's
    # stream: a table rewritten on that stream between two calls is honoured.
    wl = W.random_case(63, batch=3, H_q=8, H_kv=2, d=128, max_ctx=500)
    K, V = wl.dense_pool("cuda")
    nb = K.shape[0]
    perm = torch.from_numpy(np.random.default_rng(5).permutation(nb)).cuda()
    K2 = torch.empty_like(K)
    V2 = torch.empty_like(V)
    K2[perm] = K
    V2[perm] = V
    pool = msa.Pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, msa.BF16, k=K2, v=V2)
    try:
        bt_old = torch.from_numpy(wl.block_table.astype(np.int64)).cuda()
        bt = bt_old.to(torch.int32)                 # ids of the unpermuted pool: wrong for K2
        q = wl.q.cuda()
        desc = msa.SegDesc.from_workload(wl)
        o1 = torch.empty_like(q)
        o2 = torch.full_like(q, float("nan"))
        l2 = torch.full((wl.total_q, wl.num_q_heads), float("nan"), device="cuda")
        msa.forward(q, desc, bt, pool, o1, None)
        bt.copy_(perm[bt_old].to(torch.int32))     # enqueued on the same stream
        msa.forward(q, desc, bt, pool, o2, l2)
        torch.cuda.synchronize()
    finally:
        pool.close()
    ref_out, ref_lse = oracle_result(wl)
    compare(wl, o2.cpu(), l2.cpu(), ref_out, ref_lse)


def test_library_allocated_pool():
    wl = W.random_case(61, batch=2, H_q=8, H_kv=2, d=128)
    pool = msa.Pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, msa.BF16)
    try:
        kp, vp = pool.kv_ptrs()
        K, V = wl.dense_pool("cuda")
        torch.cuda.synchronize()
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        n = K.numel() * K.element_size()
        assert hip.hipMemcpy(kp, K.data_ptr(), n, 3) == 0 and hip.hipMemcpy(vp, V.data_ptr(), n, 3) == 0
        q = wl.q.cuda()
        out = torch.empty_like(q)
        lse = torch.empty(wl.total_q, wl.num_q_heads, device="cuda")
        bt = torch.from_numpy(wl.block_table).cuda()
        msa.forward(q, msa.SegDesc.from_workload(wl), bt, pool, out, lse)
        torch.cuda.synchronize()
    finally:
        pool.close()
    ref_out, ref_lse = oracle_result(wl)
    compare(wl, out.cpu(), lse.cpu(), ref_out, ref_lse)


# ---- benchmark configurations at full size, every row ----------------------
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_benchmark_config_full_size(cfg):
    """Every query row and head of the configuration, in the launch
    configuration the benchmark times, against the oracle."""
    wl = W.CONFIGS[cfg]()
    _check(wl)
    m = compare.last
    print(f"[parity] config {cfg} ({wl.name}): rows {m['rows']}, out max-abs {m['out_max_abs']:.3e} "
          f"mean-abs {m['out_mean_abs']:.3e}, lse max-abs {m['lse_max_abs']:.3e} mean-abs {m['lse_mean_abs']:.3e}",
          flush=True)


def test_block_id_check_option():
    """MSA_OPT_CHECK_BLOCK_IDS: a table of valid ids gives the usual result; an
    entry outside [0, num_blocks) fails the call with MSA_ERR_INVALID_ARG
    naming the first bad block-table index, for msa_forward and
    msa_forward_noalloc, before any attention kernel writes out.  Without the
    option the same table is clamped on the device and the call succeeds."""
    wl = W.random_case(64, batch=3, H_q=8, H_kv=2, d=128, max_ctx=500)
    case = GpuCase(wl)
    try:
        case.pool.set_option(msa.OPT_CHECK_BLOCK_IDS, 1)
        out, lse = case.run()
        ref_out, ref_lse = oracle_result(wl)
        compare(wl, out, lse, ref_out, ref_lse)
        used = sorted({int(s[2]) for s in wl.segs if s[1] > 0})
        bad_idx = used[len(used) // 2]
        for bad in (wl.num_blocks, -1, 1 << 27):
            bt = case.bt.clone()
            bt[bad_idx] = bad
            bt[used[-1]] = wl.num_blocks + 7
            for fn in (msa.forward, msa.forward_noalloc):
                case.out.fill_(float("nan"))
                with pytest.raises(msa.MsaError) as ei:
                    fn(case.q, case.desc, bt, case.pool, case.out, case.lse)
                torch.cuda.synchronize()
                assert ei.value.code == msa.ERR_INVALID_ARG
                assert f"block_table[{min(bad_idx, used[-1])}]" in str(ei.value), str(ei.value)
                assert torch.isnan(case.out.float()).all(), "an attention kernel ran after the failed check"
        case.pool.set_option(msa.OPT_CHECK_BLOCK_IDS, 0)
        msa.forward(case.q, case.desc, bt, case.pool, case.out, case.lse)
        torch.cuda.synchronize()
    finally:
        case.close()
