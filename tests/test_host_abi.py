"""Host-side tests of libmsa: exports, argument checks and the planner.

None of these makes a compute call: argument checks run before any HIP call,
and the planner is reachable on its own through msa_plan_debug.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_attention_msa_amd as msa
import workloads as W

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "msa.h")


def test_library_exports_every_declared_symbol():
    lib = msa.load_library()
    text = "".join(open(os.path.join(os.path.dirname(HEADER), h)).read()
                   for h in ("msa.h", "msa_latency.h", "msa_evict.h"))
    declared = set(re.findall(r"^(?:int|const char\*)\s+(msa_\w+)\s*\(", text, flags=re.M))
    assert declared == set(msa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_peaks_library_exports_its_header():
    import ctypes as ct
    path = os.path.join(os.path.dirname(msa.library_path()), "libmsa_peaks.so")
    lib = ct.CDLL(path)
    text = open(os.path.join(os.path.dirname(HEADER), "msa_peaks.h")).read()
    declared = set(re.findall(r"^int\s+(msa_\w+)\s*\(", text, flags=re.M))
    assert declared == {"msa_peak_hbm_read", "msa_peak_hbm_copy", "msa_peak_hbm_gather", "msa_peak_mfma_bf16"}
    for name in declared:
        assert hasattr(lib, name), name


def _fake_pool(num_kv_heads=2, head_dim=64, dtype=msa.BF16, num_blocks=64):
    # caller-owned pointers that are never dereferenced on the host
    lib = msa.load_library()
    desc = msa._PoolDesc(num_blocks, 16, num_kv_heads, head_dim, dtype, 0)
    h = ctypes.c_void_p()
    rc = lib.msa_create_pool(ctypes.byref(desc), 0x10000, 0x20000, ctypes.byref(h))
    assert rc == 0
    return h


def _call(h, desc, q=0x1000, bt=0x2000, out=0x3000, lse=0x4000):
    lib = msa.load_library()
    return lib.msa_forward(q, ctypes.byref(desc.c), bt, h, out, lse, 0)


def _desc(segs_per_seq, qpos_per_seq, Hq=4, bt_len=64, **kw):
    q_off, s_off, segs, qp = [0], [0], [], []
    for s, p in zip(segs_per_seq, qpos_per_seq):
        segs.extend(s)
        qp.extend(p)
        q_off.append(len(qp))
        s_off.append(len(segs))
    return msa.SegDesc(q_off, qp, s_off, np.array(segs, dtype=np.int32).reshape(-1, 4), bt_len, Hq, **kw)


GOOD = ([[(0, 20, 0, 0), (30, 5, 2, 1)]], [[34, 35]])


def test_valid_descriptor_passes_checks_on_planner():
    items, blocks = msa.plan_debug(_desc(*GOOD), 2, 64)
    assert len(blocks) == 3 and len(items) == 2


@pytest.mark.parametrize("mutate,code", [
    (lambda s, p, kw: kw.update(Hq=3), msa.ERR_INVALID_ARG),               # H_q % H_kv != 0
    (lambda s, p, kw: kw.update(Hq=2 * 129), msa.ERR_UNSUPPORTED),         # GQA ratio > 128
    (lambda s, p, kw: s[0].__setitem__(0, (0, -1, 0, 0)), msa.ERR_INVALID_ARG),   # negative len
    (lambda s, p, kw: s[0].__setitem__(0, (-5, 3, 0, 0)), msa.ERR_INVALID_ARG),   # negative position
    (lambda s, p, kw: s[0].__setitem__(1, (10, 5, 2, 0)), msa.ERR_INVALID_ARG),   # overlap
    (lambda s, p, kw: s[0].__setitem__(1, (30, 5, 64, 0)), msa.ERR_INVALID_ARG),  # bt past the table
    (lambda s, p, kw: kw.update(bt_len=2), msa.ERR_INVALID_ARG),           # table too short
    (lambda s, p, kw: kw.update(causal=2), msa.ERR_INVALID_ARG),
    (lambda s, p, kw: kw.update(scale=float("nan")), msa.ERR_INVALID_ARG),
    (lambda s, p, kw: s[0].__setitem__(0, (2**31 - 10, 20, 0, 0)), msa.ERR_INVALID_ARG),  # position overflow
])
def test_argument_checks(mutate, code):
    segs = [list(x) for x in GOOD[0]]
    qp = [list(x) for x in GOOD[1]]
    kw = {}
    mutate(segs, qp, kw)
    causal = kw.pop("causal", 1)
    d = _desc(segs, qp, **kw)
    d.c.causal = causal
    h = _fake_pool()
    try:
        assert _call(h, d) == code
        assert msa.load_library().msa_last_error().decode() != ""
    finally:
        msa.load_library().msa_destroy_pool(h)


def test_pointer_checks():
    h = _fake_pool()
    d = _desc(*GOOD)
    lib = msa.load_library()
    try:
        assert _call(h, d, q=0) == msa.ERR_INVALID_ARG
        assert _call(h, d, out=0) == msa.ERR_INVALID_ARG
        assert _call(h, d, bt=0) == msa.ERR_INVALID_ARG
        assert _call(h, d, q=0x5000, out=0x5000) == msa.ERR_INVALID_ARG   # aliasing
        assert lib.msa_forward(0x1000, None, 0x2000, h, 0x3000, 0, 0) == msa.ERR_INVALID_ARG
        assert lib.msa_forward(0x1000, ctypes.byref(d.c), 0x2000, None, 0x3000, 0, 0) == msa.ERR_INVALID_ARG
        # decreasing offsets
        bad = msa.SegDesc([0, 2, 1], [1, 2], [0, 1, 2], np.zeros((2, 4)), 8, 4)
        assert _call(h, bad) == msa.ERR_INVALID_ARG
        # empty batch: nothing to do, no HIP call
        empty = msa.SegDesc([0], [], [0], np.zeros((0, 4)), 0, 4)
        assert _call(h, empty, q=0, bt=0, out=0, lse=0) == 0
        # sequences with no query rows need no pointers either
        noq = msa.SegDesc([0, 0], [], [0, 1], np.array([[0, 5, 0, 0]]), 1, 4)
        assert _call(h, noq, q=0, out=0) == 0
    finally:
        lib.msa_destroy_pool(h)


def test_pool_creation_checks():
    lib = msa.load_library()
    h = ctypes.c_void_p()
    for nb, bs, hkv, d, dt, code in [(0, 16, 1, 64, 0, msa.ERR_INVALID_ARG), (8, 32, 1, 64, 0, msa.ERR_UNSUPPORTED),
                                     (8, 16, 1, 96, 0, msa.ERR_UNSUPPORTED), (8, 16, 1, 64, 7, msa.ERR_UNSUPPORTED),
                                     (8, 16, 0, 64, 0, msa.ERR_INVALID_ARG)]:
        desc = msa._PoolDesc(nb, bs, hkv, d, dt, 0)
        assert lib.msa_create_pool(ctypes.byref(desc), 0x10, 0x20, ctypes.byref(h)) == code
    desc = msa._PoolDesc(8, 16, 1, 64, 0, 0)
    assert lib.msa_create_pool(ctypes.byref(desc), 0x10, None, ctypes.byref(h)) == msa.ERR_INVALID_ARG
    assert lib.msa_destroy_pool(None) == 0
    h = _fake_pool()
    assert lib.msa_pool_set_option(h, msa.OPT_SPLIT_BLOCKS, 4) == 0
    assert lib.msa_pool_set_option(h, 99, 1) == msa.ERR_INVALID_ARG
    # phase tracing exists only in the measurement build (libmsa_trace.so)
    assert lib.msa_pool_set_option(h, msa.OPT_PHASE_TRACE, 0x1000) == msa.ERR_UNSUPPORTED
    assert "tracing build" in lib.msa_last_error().decode()
    assert lib.msa_pool_set_option(h, msa.OPT_PHASE_TRACE, 0) == 0
    for w, code in ((0, 0), (4, 0), (8, 0), (5, msa.ERR_INVALID_ARG), (16, msa.ERR_INVALID_ARG)):
        assert lib.msa_pool_set_option(h, msa.OPT_CHUNK_WAVES, w) == code
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.msa_pool_kernel_time(h, 0, ctypes.byref(ms), ctypes.byref(n), 1) == 0 and n.value == 0
    assert lib.msa_destroy_pool(h) == 0


# ---------------------------------------------------------------------------
# planner: exact coverage of the visible (row, head, key) set
# ---------------------------------------------------------------------------
def check_plan(wl, num_cus=256, split_blocks=0):
    d = msa.SegDesc.from_workload(wl)
    dt = msa.FP32 if wl.dtype == "fp32" else msa.BF16
    items, blocks = msa.plan_debug(d, wl.num_kv_heads, wl.head_dim, dt, num_cus, split_blocks)
    g = wl.num_q_heads // wl.num_kv_heads
    # block list matches the segments, in position order per sequence
    seq_blocks = {}
    for b in range(wl.batch):
        exp = []
        for (p0, ln, bt0, _f) in sorted(wl.seg_list(b)):
            for j in range(-(-ln // 16)):
                exp.append((bt0 + j, p0 + 16 * j, min(16, ln - 16 * j)))
        seq_blocks[b] = exp
    flat = [x for b in range(wl.batch) for x in seq_blocks[b]]
    assert [tuple(x) for x in blocks] == flat
    # coverage
    seen = {}
    parts = []
    for it in items:
        b = it["seq"]
        rows = range(it["q_row0"], it["q_row0"] + it["n_q"])
        assert wl.q_offsets[b] <= it["q_row0"] and it["q_row0"] + it["n_q"] <= wl.q_offsets[b + 1]
        qmax = max(wl.q_pos[r] for r in rows)
        if it["part_row"] >= 0:
            parts.append((it["part_row"], it["n_q"] * g))
        for bi in range(it["blk_begin"], it["blk_end"]):
            bt, p0, valid = blocks[bi]
            if wl.causal:
                assert p0 <= qmax, "a fully masked block was scheduled"
            for r in rows:
                for s in range(valid):
                    if not wl.causal or p0 + s <= wl.q_pos[r]:
                        key = (r, it["kv_head"], p0 + s)
                        seen[key] = seen.get(key, 0) + 1
        expect_kind = msa.KERNEL_FP32 if wl.dtype == "fp32" else None
        if expect_kind is not None:
            assert it["kind"] == expect_kind
    expected = set()
    for b in range(wl.batch):
        kpos = [p0 + s for (_bt, p0, valid) in seq_blocks[b] for s in range(valid)]
        for r in range(wl.q_offsets[b], wl.q_offsets[b + 1]):
            for h in range(wl.num_kv_heads):
                for p in kpos:
                    if not wl.causal or p <= wl.q_pos[r]:
                        expected.add((r, h, p))
    assert set(seen) == expected
    assert all(c == 1 for c in seen.values())
    # every (row, kv head) tile appears, including rows that see nothing
    covered_rows = {(r, it["kv_head"]) for it in items for r in range(it["q_row0"], it["q_row0"] + it["n_q"])}
    assert covered_rows == {(r, h) for r in range(wl.total_q) for h in range(wl.num_kv_heads)}
    # partial rows are disjoint
    parts.sort()
    for (a0, an), (b0, _bn) in zip(parts, parts[1:]):
        assert a0 + an <= b0
    return items, blocks


@pytest.mark.parametrize("seed", range(8))
def test_planner_exact_coverage_random(seed):
    wl = W.random_case(seed, batch=4, H_q=8, H_kv=2, d=64, max_ctx=200, max_chunk=50)
    check_plan(wl)
    check_plan(wl, split_blocks=3)
    check_plan(wl, num_cus=2)


def test_planner_exact_coverage_fp32_and_noncausal():
    wl = W.config1()
    check_plan(wl)
    check_plan(wl, split_blocks=1)
    wl2 = W.custom([([(0, 40), (100, 7)], [5, 50, 200]), ([], [3]), ([(10, 3)], [])], H_q=2, H_kv=2,
                   d=64, causal=0)
    check_plan(wl2, split_blocks=2)


def test_planner_ordered_and_shuffled_segments_agree():
    # the planner sorts a sequence's segments only when they arrive out of
    # position order; both inputs must give the same block list and items
    spec = [([(0, 40), (48, 33), (100, 7), (300, 64)], [10, 120, 363]), ([(5, 17), (30, 1)], [30])]
    plans = []
    for shuffle in (False, True):
        wl = W.custom(spec, H_q=4, H_kv=2, d=64, shuffle=shuffle, seed=3)
        if not shuffle:
            for b in range(wl.batch):
                p = wl.segs[wl.seg_offsets[b]:wl.seg_offsets[b + 1], 0]
                assert list(p) == sorted(p)
        items, blocks = check_plan(wl, split_blocks=2)
        plans.append(([(p0, v) for (_bt, p0, v) in blocks], sorted(
            (int(it["kv_head"]), int(it["q_row0"]), int(it["blk_begin"]), int(it["blk_end"])) for it in items)))
    assert plans[0] == plans[1]


def test_planner_kinds_and_lpt_order():
    wl = W.custom([([(0, 100)], [99]), ([(0, 300)], list(range(300, 340)))], H_q=8, H_kv=2, d=128)
    items, _ = check_plan(wl)
    kinds = {(it["seq"], it["kind"]) for it in items}
    assert (0, msa.KERNEL_DECODE) in kinds and (1, msa.KERNEL_PREFILL) in kinds
    for k in (msa.KERNEL_PREFILL, msa.KERNEL_DECODE):
        sizes = [it["blk_end"] - it["blk_begin"] for it in items if it["kind"] == k]
        assert sizes == sorted(sizes, reverse=True)


def check_plan_ranges(wl, num_cus=256):
    """Cheaper check for large plans: per (query tile, kv head) the items' block
    ranges tile [first block of the sequence, first block past the tile's
    largest position) without gaps or overlap."""
    d = msa.SegDesc.from_workload(wl)
    items, blocks = msa.plan_debug(d, wl.num_kv_heads, wl.head_dim, msa.BF16, num_cus, 0)
    pos0 = blocks["pos0"]
    seq_start = {}
    off = 0
    for b in range(wl.batch):
        seq_start[b] = off
        off += int(sum(-(-int(x) // 16) for x in wl.segs[wl.seg_offsets[b]:wl.seg_offsets[b + 1], 1]))
    tiles = {}
    for it in items:
        tiles.setdefault((int(it["seq"]), int(it["q_row0"]), int(it["n_q"]), int(it["kv_head"])), []).append(
            (int(it["blk_begin"]), int(it["blk_end"])))
    rows = set()
    for (b, r0, n, h), rng in tiles.items():
        rng.sort()
        qmax = int(wl.q_pos[r0:r0 + n].max())
        nxt = seq_start[b + 1] if b + 1 in seq_start else off
        end = seq_start[b] + int(np.searchsorted(pos0[seq_start[b]:nxt], qmax, side="right"))
        assert rng[0][0] == seq_start[b] and rng[-1][1] == end
        for (a0, a1), (b0, _b1) in zip(rng, rng[1:]):
            assert a1 == b0
        rows.update((r, h) for r in range(r0, r0 + n))
    assert rows == {(r, h) for r in range(wl.total_q) for h in range(wl.num_kv_heads)}


def test_planner_on_benchmark_configs():
    check_plan(W.CONFIGS[1]())
    for i in (2, 4):
        check_plan_ranges(W.CONFIGS[i]())


def test_planner_split_alignment():
    wl = W.custom([([(0, 2000)], list(range(1900, 2000)))], H_q=4, H_kv=1, d=128)
    items, blocks = check_plan(wl, split_blocks=10)
    pre = [it for it in items if it["kind"] == msa.KERNEL_PREFILL]
    assert len(pre) > 1
    for it in pre:
        starts = {x["blk_begin"] for x in pre if x["q_row0"] == it["q_row0"]}
        assert all((s - min(starts)) % 4 == 0 for s in starts)


def _write(h, segs, src_rows, n_rows=100, bt_len=32, k=0x10000000, v=0x20000000, bt=0x2000):
    lib = msa.load_library()
    segs = np.ascontiguousarray(np.asarray(segs, dtype=np.int32).reshape(-1, 4))
    src = np.ascontiguousarray(src_rows, dtype=np.int32)
    return lib.msa_write_kv(h, k, v, n_rows, segs.ctypes.data if len(segs) else None,
                            src.ctypes.data if len(src) else None, len(segs), bt, bt_len, 0)


def test_write_kv_argument_checks():
    """Every msa_write_kv check runs before a HIP call, so these need no GPU."""
    h = _fake_pool()
    lib = msa.load_library()
    E = msa.ERR_INVALID_ARG
    try:
        assert _write(h, [], []) == msa.OK                                  # nothing to write
        assert _write(h, [(0, 0, 0, 1)], [0]) == msa.OK                     # only empty segments
        assert _write(h, [(0, -1, 0, 1)], [0]) == E                         # negative len
        assert _write(h, [(0, 5, -1, 1)], [0]) == E                         # negative bt_start
        assert _write(h, [(0, 5, 0, 1)], [-1]) == E                         # negative source row
        assert _write(h, [(0, 33, 30, 1)], [0]) == E                        # bt range 30..33 > 32 entries
        assert _write(h, [(0, 20, 0, 1)], [81]) == E                        # rows 81..101 > 100
        assert _write(h, [(0, 20, 0, 1), (50, 5, 1, 1)], [0, 40]) == E      # both use bt entry 1
        assert _write(h, [(0, 20, 0, 1)], [0], k=0) == E                    # null source
        assert _write(h, [(0, 20, 0, 1)], [0], bt=0) == E                   # null block table
        assert _write(h, [(0, 20, 0, 1)], [0], v=0x10000000) == E           # k_src == v_src
        assert _write(h, [(0, 20, 0, 1)], [0], k=0x18000) == E              # source inside the pool
        assert lib.msa_write_kv(None, 1, 2, 10, None, None, 0, 3, 4, 0) == E
        assert lib.msa_write_kv(h, 1, 2, 10, None, None, 1, 3, 4, 0) == E   # segs NULL with num_segs 1
        assert lib.msa_write_kv(h, 1, 2, -1, None, None, 0, 3, 4, 0) == E
        assert _write(h, [(0, 20, 0, 1), (50, 5, 1, 1)], [0, 40]) == E
        assert "block-table entry 1" in lib.msa_last_error().decode()
    finally:
        lib.msa_destroy_pool(h)


def test_kernel_time_and_samples_argument_checks():
    h = _fake_pool()
    lib = msa.load_library()
    try:
        ms, n = ctypes.c_double(), ctypes.c_int64()
        assert lib.msa_pool_kernel_time(h, 99, ctypes.byref(ms), ctypes.byref(n), 0) == msa.ERR_INVALID_ARG
        assert lib.msa_pool_kernel_time(h, msa.KERNEL_PREFILL, ctypes.byref(ms), ctypes.byref(n), 0) == msa.OK
        assert ms.value == 0.0 and n.value == 0
        out = np.zeros(4)
        cnt = ctypes.c_int32(-1)
        assert lib.msa_pool_kernel_samples(h, msa.KERNEL_DECODE, out.ctypes.data, 4, ctypes.byref(cnt)) == msa.OK
        assert cnt.value == 0
        assert lib.msa_pool_kernel_samples(h, -1, out.ctypes.data, 4, ctypes.byref(cnt)) == msa.ERR_INVALID_ARG
        assert lib.msa_pool_kernel_samples(h, 0, None, 4, ctypes.byref(cnt)) == msa.ERR_INVALID_ARG
        assert lib.msa_pool_kernel_samples(h, 0, out.ctypes.data, -1, ctypes.byref(cnt)) == msa.ERR_INVALID_ARG
        assert lib.msa_pool_kernel_samples(h, 0, out.ctypes.data, 4, None) == msa.ERR_INVALID_ARG
        assert lib.msa_pool_set_option(h, 77, 1) == msa.ERR_INVALID_ARG
    finally:
        lib.msa_destroy_pool(h)


def test_binding_checks_tensor_shapes_before_the_library():
    # The C ABI gets bare pointers; the Python binding rejects tensors whose
    # shape, dtype, layout or device cannot match the descriptor, before any
    # library call (a pool stand-in with the attributes the check reads).
    import types
    import torch
    d = msa.SegDesc([0, 3], [5, 6, 7], [0, 1], [[0, 8, 0, 0]], 1, num_q_heads=4)
    pool = types.SimpleNamespace(head_dim=64, dtype=msa.BF16, handle=None)
    good_q = torch.zeros(3, 4, 64, dtype=torch.bfloat16)        # right shape, but host memory
    with pytest.raises(ValueError, match="q must be"):
        msa.forward(good_q, d, 0x2000, pool, 0x3000)
    with pytest.raises(ValueError, match="out must be"):
        msa.forward(0x1000, d, 0x2000, pool, torch.zeros(3, 4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must be"):
        msa.forward(0x1000, d, 0x2000, pool, 0x3000, torch.zeros(3, 5))
    with pytest.raises(ValueError, match="block_table must be"):
        msa.forward(0x1000, d, torch.zeros(1, dtype=torch.int64), pool, 0x3000)


def test_chunk_work_group_size_choice():
    """The planner takes 8-wave work-groups (256-row tiles) only for a
    prefill-only batch with at least two such tiles per compute unit and long
    contexts: the heavy-fragmentation workload; the prefill and mixed
    workloads keep 128-row tiles."""
    for wl, rows in ((W.config2(), 128), (W.config4(), 256), (W.config5(), 128)):
        group = wl.num_q_heads // wl.num_kv_heads
        items, _ = msa.plan_debug(msa.SegDesc.from_workload(wl), wl.num_kv_heads, wl.head_dim)
        chunk = items[items["launch"] == msa.KERNEL_PREFILL]
        assert int((chunk["n_q"] * group).max()) == rows, wl.name
