"""Calibrate the Eq. 5 latency model of the AsymCache / Multi-Segment Attention
paper (Figure 6 caption) against this library on the current GPU.

The pages give the marginal cost of recomputing one block instead of keeping
it cached, dT_B = k5 (l1 + 2 q1) + (k2 - k3 + k5), with coefficients that
depend on the hardware.  ``measure_grid`` times one serving step of a batch of
requests shaped (l1 cached | q1 recomputed | l2 cached | q2 new) blocks --
the KV write of the q1 + q2 fresh blocks followed by MSA for their query rows
-- over a grid of shapes; ``calibrate`` fits k1..k5 to those times with the
library's native fitter (include/msa_latency.h).  Every step runs in libmsa's
kernels; torch only provides device memory, random contents and events.
"""
from __future__ import annotations

import itertools

import numpy as np

from . import BF16, BLOCK_SIZE, SEG_FRESH, Pool, SegDesc, forward, latency_fit, write_kv

DEFAULT_GRID = {"l1": (0, 64, 128, 256), "q1": (0, 8, 32, 64), "l2": (0, 64, 256), "q2": (1, 8, 32)}


def request_layout(l1, q1, l2, q2):
    """Segments (pos_start, len, flags) and query positions of one request whose
    regions, in position order, are l1 cached, q1 recomputed, l2 cached and q2
    new blocks.  Recomputed and new blocks are fresh and carry query rows."""
    segs, qpos, pos = [], [], 0
    for n, fresh in ((l1, False), (q1, True), (l2, False), (q2, True)):
        tokens = int(n) * BLOCK_SIZE
        if tokens:
            segs.append((pos, tokens, SEG_FRESH if fresh else 0))
            if fresh:
                qpos.extend(range(pos, pos + tokens))
        pos += tokens
    return segs, qpos


class _Bench:
    def __init__(self, batch, num_kv_heads, group, head_dim, max_blocks, seed):
        import torch
        self.torch = torch
        self.batch, self.H_kv, self.H_q, self.d = batch, num_kv_heads, num_kv_heads * group, head_dim
        self.num_blocks = batch * max_blocks
        g = torch.Generator(device="cuda").manual_seed(seed)
        shape = (self.num_blocks, num_kv_heads, BLOCK_SIZE, head_dim)
        self.K = (torch.randn(shape, generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        self.V = (torch.randn(shape, generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        self.pool = Pool(self.num_blocks, num_kv_heads, head_dim, BF16, k=self.K, v=self.V)
        max_rows = batch * max_blocks * BLOCK_SIZE
        self.q = (torch.randn((max_rows, self.H_q, head_dim), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((max_rows, self.H_q), dtype=torch.float32, device="cuda")
        self.k_src = (torch.randn((max_rows, num_kv_heads, head_dim), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        self.v_src = torch.randn_like(self.k_src)
        self.rng = np.random.default_rng(seed)

    def step_inputs(self, l1, q1, l2, q2):
        segs, qpos_all, seg_off, q_off = [], [], [0], [0]
        fresh, src_rows = [], []
        bt_len, src = 0, 0
        for _ in range(self.batch):
            s, qp = request_layout(l1, q1, l2, q2)
            for pos, n, flags in s:
                seg = (pos, n, bt_len, flags)
                segs.append(seg)
                if flags & SEG_FRESH:
                    fresh.append(seg)
                    src_rows.append(src)
                    src += n
                bt_len += -(-n // BLOCK_SIZE)
            qpos_all.extend(qp)
            seg_off.append(len(segs))
            q_off.append(len(qpos_all))
        bt = self.rng.permutation(self.num_blocks)[:bt_len].astype(np.int32)
        desc = SegDesc(q_off, qpos_all, seg_off, np.array(segs, dtype=np.int32).reshape(-1, 4), bt_len, self.H_q)
        return desc, self.torch.from_numpy(bt).cuda(), np.array(fresh, dtype=np.int32).reshape(-1, 4), \
            np.array(src_rows, dtype=np.int32), src

    def time(self, l1, q1, l2, q2, reps, warmup):
        torch = self.torch
        desc, bt, fresh, src_rows, n_src = self.step_inputs(l1, q1, l2, q2)
        ks, vs = self.k_src[:n_src], self.v_src[:n_src]
        stream = torch.cuda.current_stream()

        def step():
            write_kv(self.pool, ks, vs, fresh, src_rows, bt, stream)
            forward(self.q, desc, bt, self.pool, self.out, self.lse, stream)

        for _ in range(warmup):
            step()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3   # microseconds

    def settle(self, l1, q1, l2, q2, seconds):
        """Back-to-back steps until the GPU has been busy for `seconds`, so that
        the first grid points are not timed while its clocks are still rising
        from idle."""
        import time
        torch = self.torch
        desc, bt, fresh, src_rows, n_src = self.step_inputs(l1, q1, l2, q2)
        ks, vs = self.k_src[:n_src], self.v_src[:n_src]
        stream = torch.cuda.current_stream()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                write_kv(self.pool, ks, vs, fresh, src_rows, bt, stream)
                forward(self.q, desc, bt, self.pool, self.out, self.lse, stream)
            torch.cuda.synchronize()

    def close(self):
        self.pool.close()


def measure_grid(grid=None, batch=8, num_kv_heads=8, group=4, head_dim=128, reps=15, warmup=3, seed=0,
                 extra_points=()):
    """Median device time (us) of one step for every (l1, q1, l2, q2) of the grid
    (a dict of value lists, sizes in blocks) plus ``extra_points``.  Returns an
    array of rows (l1, q1, l2, q2, T_us)."""
    grid = grid or DEFAULT_GRID
    pts = list(itertools.product(grid["l1"], grid["q1"], grid["l2"], grid["q2"])) + list(extra_points)
    pts = [p for p in pts if p[1] + p[3] > 0]
    max_blocks = max(sum(p) for p in pts)
    bench = _Bench(batch, num_kv_heads, group, head_dim, max_blocks, seed)
    try:
        bench.settle(*max(pts, key=sum), seconds=0.3)
        rows = [(*p, bench.time(*p, reps=reps, warmup=warmup)) for p in pts]
    finally:
        bench.close()
    return np.array(rows, dtype=np.float64)


def calibrate(samples, relative=True):
    """Fit k1..k5 (microseconds per block / block^2) to measured rows."""
    return latency_fit(samples, relative=relative)
