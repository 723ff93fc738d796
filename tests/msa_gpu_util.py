"""Helpers for GPU parity tests: run a workload through libmsa and through the oracle."""
import numpy as np
import torch

import kv_cache_attention_msa_amd as msa
from oracle import attend

BF16_MAX_ABS = 2e-2    # bf16 inputs: max-abs error bound on out (and lse)
BF16_MEAN_ABS = 2e-3   # bf16 inputs: mean-abs error bound
FP32_MAX_ABS = 1e-5    # fp32 inputs: max-abs error bound


class GpuCase:
    """A workload resident on the GPU, with a pool wrapping its K/V."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.K, self.V = wl.dense_pool(device)
        dt = msa.FP32 if wl.dtype == "fp32" else msa.BF16
        self.pool = msa.Pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, dt, k=self.K, v=self.V)
        self.q = wl.q.to(device)
        self.bt = torch.from_numpy(wl.block_table.astype(np.int32)).to(device)
        if self.bt.numel() == 0:
            self.bt = torch.zeros(1, dtype=torch.int32, device=device)
        self.desc = msa.SegDesc.from_workload(wl)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(wl.total_q, wl.num_q_heads, dtype=torch.float32, device=device)

    def run(self, split_blocks=0, sync=True, chunk_waves=0):
        self.pool.set_option(msa.OPT_SPLIT_BLOCKS, split_blocks)
        self.pool.set_option(msa.OPT_CHUNK_WAVES, chunk_waves)
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        msa.forward(self.q, self.desc, self.bt, self.pool, self.out, self.lse)
        if sync:
            torch.cuda.synchronize()
        return self.out.cpu(), self.lse.cpu()

    def close(self):
        self.pool.close()


def oracle_result(wl, rows=None):
    Kp, Vp = wl.sparse_pools_f64()
    return attend(wl.q_f64(), wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, wl.block_table, Kp, Vp,
                  wl.num_kv_heads, scale=wl.scale, causal=bool(wl.causal), rows=rows)


def compare(wl, out, lse, ref_out, ref_lse, rows=None):
    """Assert the GPU result matches the oracle within the dtype's bound.

    Returns (max_abs, mean_abs) of the output error; the lse margins of the
    last call are left in ``compare.last`` (a dict of all four figures)."""
    if rows is None:
        rows = np.arange(wl.total_q)
    rows = np.asarray(rows)
    o = out.to(torch.float64).numpy()[rows]
    r = ref_out[rows]
    assert np.isfinite(o).all(), "non-finite output"
    err = np.abs(o - r)
    g_l = lse.to(torch.float64).numpy()[rows]
    r_l = ref_lse[rows]
    assert np.array_equal(np.isneginf(g_l), np.isneginf(r_l)), "rows without visible keys differ"
    fin = np.isfinite(r_l)
    assert np.isfinite(g_l[fin]).all()
    lerr = np.abs(g_l[fin] - r_l[fin])
    if wl.dtype == "fp32":
        assert err.max(initial=0) <= FP32_MAX_ABS, err.max()
        assert lerr.max(initial=0) <= FP32_MAX_ABS, lerr.max()
    else:
        assert err.max(initial=0) <= BF16_MAX_ABS, err.max()
        assert err.mean() <= BF16_MEAN_ABS, err.mean()
        assert lerr.max(initial=0) <= BF16_MAX_ABS, lerr.max()
        if lerr.size:
            assert lerr.mean() <= BF16_MEAN_ABS, lerr.mean()
    compare.last = {"rows": int(len(rows)),
                    "out_max_abs": float(err.max(initial=0)), "out_mean_abs": float(err.mean()) if err.size else 0.0,
                    "lse_max_abs": float(lerr.max(initial=0)), "lse_mean_abs": float(lerr.mean()) if lerr.size else 0.0}
    return compare.last["out_max_abs"], compare.last["out_mean_abs"]


def sample_rows(wl, n, seed):
    """A seeded sample of query rows, always including each sequence's first and last row."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(wl.batch):
        if wl.q_offsets[b + 1] > wl.q_offsets[b]:
            rows.add(int(wl.q_offsets[b]))
            rows.add(int(wl.q_offsets[b + 1] - 1))
    extra = rng.choice(wl.total_q, size=min(n, wl.total_q), replace=False)
    rows.update(int(x) for x in extra)
    return np.array(sorted(rows))
