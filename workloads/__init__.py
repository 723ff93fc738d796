"""Seeded synthetic inputs for Multi-Segment Attention.

This module only *draws* inputs: block-paged K/V pools, segment descriptors,
block tables, query positions and query vectors.  It holds none of the
attention arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``kv_cache_attention_msa_amd``) can be fed from it without sharing code.

Layout of what is drawn (one sequence = one request in a serving batch):

* K/V pool: ``[num_blocks][H_kv][block_size][d]``; only blocks referenced by a
  segment get values, every other slot (whole unused blocks and the tail
  slots of a partially filled last block) holds NaN, so that any read outside
  the segments shows up in the result.
* A segment is ``(pos_start, len, bt_start, flags)``: token ``i < len`` has
  absolute position ``pos_start + i`` and lives in pool block
  ``block_table[bt_start + i // block_size]``, slot ``i % block_size``.
  ``flags`` bit 0 marks K/V written in this step (recomputed or new); it
  carries no numerical meaning.
* ``seg_offsets[b]:seg_offsets[b+1]`` are sequence ``b``'s segments and
  ``q_offsets[b]:q_offsets[b+1]`` its query rows; ``q_pos`` holds each query
  row's absolute position.

The multi-segment setting (a cached prefix and a cached suffix, with evicted
blocks recomputed on demand, attended in one launch) is the one described on
the AsymCache / Multi-Segment Attention page (section 4.1 and the Eq. 5
layout of l1, q1, l2, q2 regions).  Configurations 1-5 follow the five
synthetic workloads of the benchmark definition; value distributions that the
workload definitions leave open are N(0,1)*0.5 rounded to bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

BLOCK_SIZE = 16
SEG_FRESH = 1  # flags bit 0: K/V written in this step (recomputed or new)


# --------------------------------------------------------------------------
# container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    dtype: str                      # "fp32" | "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    q: torch.Tensor                 # [total_q, H_q, d] (CPU, dtype)
    k_blocks: torch.Tensor          # [n_used, H_kv, bs, d] (CPU, dtype), NaN tails
    v_blocks: torch.Tensor
    used_ids: np.ndarray            # [n_used] int64 physical block ids
    q_offsets: np.ndarray           # [B+1] int32
    q_pos: np.ndarray               # [total_q] int32
    seg_offsets: np.ndarray         # [B+1] int32
    segs: np.ndarray                # [n_segs, 4] int32 (pos_start, len, bt_start, flags)
    block_table: np.ndarray         # [bt_len] int32
    scale: float = 0.0              # 0 -> 1/sqrt(head_dim)
    causal: int = 1
    block_size: int = BLOCK_SIZE
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.q_offsets) - 1

    @property
    def total_q(self) -> int:
        return int(self.q_offsets[-1])

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    # ---- pools -----------------------------------------------------------
    def dense_pool(self, device="cpu"):
        """Full K and V pools with NaN in every slot no segment covers."""
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        K = torch.full(shape, float("nan"), dtype=self.torch_dtype, device=device)
        V = torch.full(shape, float("nan"), dtype=self.torch_dtype, device=device)
        if len(self.used_ids):
            idx = torch.from_numpy(self.used_ids).to(device)
            K[idx] = self.k_blocks.to(device)
            V[idx] = self.v_blocks.to(device)
        return K, V

    def sparse_pools_f64(self):
        """Indexable K and V pools that materialise only what is asked for."""
        return (SparsePool(self.k_blocks, self.used_ids, self.num_blocks),
                SparsePool(self.v_blocks, self.used_ids, self.num_blocks))

    def q_f64(self) -> np.ndarray:
        return self.q.to(torch.float64).numpy()

    def seg_list(self, b):
        return [tuple(int(x) for x in s) for s in self.segs[self.seg_offsets[b]:self.seg_offsets[b + 1]]]


class SparsePool:
    """``pool[ids, :, slots, :]`` over a pool whose used blocks are stored compactly.

    Returns float64 (an exact widening of bf16/fp32); unused blocks read as NaN.
    """

    def __init__(self, blocks: torch.Tensor, used_ids: np.ndarray, num_blocks: int):
        self.blocks = blocks
        self.inv = np.full(num_blocks, -1, dtype=np.int64)
        self.inv[used_ids] = np.arange(len(used_ids))
        self.shape = (num_blocks,) + tuple(blocks.shape[1:])

    def __getitem__(self, key):
        ids, s1, slots, s2 = key
        assert s1 == slice(None) and s2 == slice(None)
        ids = np.asarray(ids, dtype=np.int64)
        slots = np.asarray(slots, dtype=np.int64)
        comp = self.inv[ids]
        out = np.full((len(ids),) + (self.shape[1], self.shape[3]), np.nan)
        ok = comp >= 0
        if ok.any():
            sel = self.blocks[torch.from_numpy(comp[ok]), :, torch.from_numpy(slots[ok]), :]
            out[ok] = sel.to(torch.float64).numpy()
        return out


# --------------------------------------------------------------------------
# builder
# --------------------------------------------------------------------------
class _Builder:
    """Allocates pool blocks for segments and records descriptors."""

    def __init__(self, rng, num_blocks, fresh_from=None):
        self.rng = rng
        self.num_blocks = num_blocks
        split = num_blocks if fresh_from is None else fresh_from
        self.cached_free = list(rng.permutation(split))
        self.fresh_free = list(split + rng.permutation(num_blocks - split)) if fresh_from is not None else None
        self.bt = []
        self.blocks = []  # (phys_id, n_valid)
        self.seqs = []    # per sequence: (segments list, q positions)

    def segment(self, pos_start, length, flags=0):
        assert length >= 0
        nb = -(-length // BLOCK_SIZE)
        pool = self.fresh_free if (flags & SEG_FRESH and self.fresh_free is not None) else self.cached_free
        if len(pool) < nb:
            raise ValueError("pool too small for requested segments")
        ids = [pool.pop() for _ in range(nb)]
        bt_start = len(self.bt)
        self.bt.extend(ids)
        for j, pid in enumerate(ids):
            self.blocks.append((pid, min(BLOCK_SIZE, length - BLOCK_SIZE * j)))
        return (pos_start, length, bt_start, flags)

    def add_sequence(self, segments, q_positions, shuffle=True):
        segments = list(segments)
        if shuffle and len(segments) > 1:
            order = self.rng.permutation(len(segments))
            segments = [segments[i] for i in order]
        self.seqs.append((segments, list(q_positions)))

    def finish(self, name, dtype, H_q, H_kv, d, qscale, kvscale, scale=0.0, causal=1, meta=None):
        tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
        rng = self.rng
        n_used = len(self.blocks)
        kv_shape = (n_used, H_kv, BLOCK_SIZE, d)
        k = torch.from_numpy(rng.standard_normal(kv_shape, dtype=np.float32) * np.float32(kvscale)).to(tdt)
        v = torch.from_numpy(rng.standard_normal(kv_shape, dtype=np.float32) * np.float32(kvscale)).to(tdt)
        for i, (_, nv) in enumerate(self.blocks):
            if nv < BLOCK_SIZE:
                k[i, :, nv:, :] = float("nan")
                v[i, :, nv:, :] = float("nan")
        used_ids = np.array([p for p, _ in self.blocks], dtype=np.int64)
        q_offsets = [0]
        seg_offsets = [0]
        segs, q_pos = [], []
        for s, qp in self.seqs:
            segs.extend(s)
            q_pos.extend(qp)
            q_offsets.append(len(q_pos))
            seg_offsets.append(len(segs))
        total_q = len(q_pos)
        q = torch.from_numpy(rng.standard_normal((total_q, H_q, d), dtype=np.float32) * np.float32(qscale)).to(tdt)
        return Workload(
            name=name, dtype=dtype, num_q_heads=H_q, num_kv_heads=H_kv, head_dim=d,
            num_blocks=self.num_blocks, q=q, k_blocks=k, v_blocks=v, used_ids=used_ids,
            q_offsets=np.array(q_offsets, dtype=np.int32),
            q_pos=np.array(q_pos, dtype=np.int32).reshape(-1),
            seg_offsets=np.array(seg_offsets, dtype=np.int32),
            segs=np.array(segs, dtype=np.int32).reshape(-1, 4),
            block_table=np.array(self.bt, dtype=np.int32),
            scale=scale, causal=causal, meta=dict(meta or {}),
        )


def _composition(rng, total, parts, unit=1):
    """Split ``total`` into ``parts`` positive multiples of ``unit`` (uniform cut points)."""
    n_units = total // unit
    assert n_units * unit == total and 1 <= parts <= n_units
    cuts = np.sort(rng.choice(np.arange(1, n_units), size=parts - 1, replace=False)) if parts > 1 else np.array([], dtype=np.int64)
    edges = np.concatenate([[0], cuts, [n_units]])
    return [int(x) * unit for x in np.diff(edges)]


def _contiguous_segments(b, sizes, start=0, fresh_mask=None):
    segs, pos = [], start
    for i, s in enumerate(sizes):
        flag = SEG_FRESH if (fresh_mask is not None and fresh_mask[i]) else 0
        segs.append(b.segment(pos, s, flag))
        pos += s
    return segs, pos


# --------------------------------------------------------------------------
# the five benchmark configurations
# --------------------------------------------------------------------------
def config1(seed=1):
    """Tiny fp32: 1 seq, 1 head, d 64, pool of 8 blocks; context segments of
    16, 32, 16 tokens (positions 0-63) at shuffled blocks; a 16-token chunk at
    positions 64-79 whose own K/V is the final (fresh) segment; causal."""
    rng = np.random.default_rng(seed)
    b = _Builder(rng, 8)
    segs, pos = _contiguous_segments(b, [16, 32, 16])
    segs.append(b.segment(pos, 16, SEG_FRESH))
    b.add_sequence(segs, range(64, 80))
    return b.finish("tiny_fp32", "fp32", 1, 1, 64, qscale=1.0, kvscale=1.0)


def config2(seed=2):
    """Chunked prefill, bf16, Llama-3-8B head shape (32 q / 8 kv heads, d 128),
    batch 4: a 4096-token context in 6 segments of whole blocks at scattered
    pool blocks, plus a 512-token chunk (positions 4096-4607) with its own K/V."""
    rng = np.random.default_rng(seed)
    B, ctx, chunk = 4, 4096, 512
    used = B * (ctx + chunk) // BLOCK_SIZE
    b = _Builder(rng, 2 * used)
    for _ in range(B):
        sizes = _composition(rng, ctx, 6, unit=BLOCK_SIZE)
        segs, pos = _contiguous_segments(b, sizes)
        segs.append(b.segment(pos, chunk, SEG_FRESH))
        b.add_sequence(segs, range(pos, pos + chunk))
    return b.finish("prefill_b4_ctx4096_chunk512", "bf16", 32, 8, 128, qscale=0.5, kvscale=0.5)


def config3(seed=3):
    """Decode, bf16, batch 64, one query token per sequence, GQA 32/8, d 128;
    contexts U{1024..8192} tokens in U{2..16} segments of arbitrary length,
    scattered over a 2M-token pool; the query is the last context token."""
    rng = np.random.default_rng(seed)
    B = 64
    b = _Builder(rng, 2 * 1024 * 1024 // BLOCK_SIZE)
    for _ in range(B):
        L = int(rng.integers(1024, 8192, endpoint=True))
        n = int(rng.integers(2, 16, endpoint=True))
        segs, _ = _contiguous_segments(b, _composition(rng, L, n))
        b.add_sequence(segs, [L - 1])
    return b.finish("decode_b64_ctx1k-8k", "bf16", 32, 8, 128, qscale=0.5, kvscale=0.5)


def _log_uniform_sizes(rng, n, total, lo, hi):
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), n))
    x = x * total / x.sum()
    s = np.clip(np.round(x), lo, hi).astype(np.int64)
    diff = int(total - s.sum())
    order = rng.permutation(n)
    while diff != 0:
        moved = False
        for i in order:
            if diff > 0 and s[i] < hi:
                s[i] += 1; diff -= 1; moved = True
            elif diff < 0 and s[i] > lo:
                s[i] -= 1; diff += 1; moved = True
            if diff == 0:
                break
        assert moved
    return [int(v) for v in s]


def config4(seed=4):
    """Heavy fragmentation, bf16, batch 2, GQA 32/8, d 128: a 32768-token
    context in 64 segments (log-uniform 16-4096 tokens) separated by position
    gaps U{1..256}; a 2048-token chunk after one more gap; causal by position."""
    rng = np.random.default_rng(seed)
    B, ctx, n, chunk = 2, 32768, 64, 2048
    b = _Builder(rng, 8192)
    for _ in range(B):
        sizes = _log_uniform_sizes(rng, n, ctx, 16, 4096)
        segs, pos = [], 0
        for s in sizes:
            segs.append(b.segment(pos, s))
            pos += s + int(rng.integers(1, 256, endpoint=True))
        segs.append(b.segment(pos, chunk, SEG_FRESH))
        b.add_sequence(segs, range(pos, pos + chunk))
    return b.finish("heavyfrag_b2_ctx32k_64segs_chunk2048", "bf16", 32, 8, 128, qscale=0.5, kvscale=0.5)


def config5(seed=5):
    """Mixed batch, bf16, 16 sequences, GQA 64/8, d 128: 8 prefill chunks of
    U{64..2048} tokens and 8 decode tokens; contexts U{2048..16384} tokens in
    U{4..32} segments, about 25% flagged fresh (recomputed, placed in a disjoint
    block range); the sequences are interleaved in random order."""
    rng = np.random.default_rng(seed)
    nb = 65536
    b = _Builder(rng, nb, fresh_from=3 * nb // 4)
    kinds = ["prefill"] * 8 + ["decode"] * 8
    kinds = [kinds[i] for i in rng.permutation(16)]
    for kind in kinds:
        L = int(rng.integers(2048, 16384, endpoint=True))
        n = int(rng.integers(4, 32, endpoint=True))
        fresh = rng.random(n) < 0.25
        segs, pos = _contiguous_segments(b, _composition(rng, L, n), fresh_mask=fresh)
        if kind == "prefill":
            c = int(rng.integers(64, 2048, endpoint=True))
            segs.append(b.segment(pos, c, SEG_FRESH))
            b.add_sequence(segs, range(pos, pos + c))
        else:
            b.add_sequence(segs, [L - 1])
    return b.finish("mixed_16seq_gqa64-8", "bf16", 64, 8, 128, qscale=0.5, kvscale=0.5,
                    meta={"kinds": kinds})


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def subset(wl, seqs, name):
    """The sequences ``seqs`` of ``wl`` (in that order) as a workload of their
    own, over the same pool and block table (e.g. the prefill-only or the
    decode-only part of the mixed batch)."""
    rows, q_pos, segs = [], [], []
    q_off, s_off = [0], [0]
    for b in seqs:
        r0, r1 = int(wl.q_offsets[b]), int(wl.q_offsets[b + 1])
        rows.append(np.arange(r0, r1, dtype=np.int64))
        q_pos.extend(wl.q_pos[r0:r1].tolist())
        segs.extend(wl.segs[wl.seg_offsets[b]:wl.seg_offsets[b + 1]].tolist())
        q_off.append(q_off[-1] + r1 - r0)
        s_off.append(len(segs))
    idx = torch.from_numpy(np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64))
    return replace(wl, name=name, q=wl.q[idx].contiguous(),
                   q_offsets=np.array(q_off, dtype=np.int32), q_pos=np.array(q_pos, dtype=np.int32).reshape(-1),
                   seg_offsets=np.array(s_off, dtype=np.int32),
                   segs=np.array(segs, dtype=np.int32).reshape(-1, 4), meta=dict(wl.meta, subset_of=wl.name))


def mixed_parts(wl):
    """Sequence indices of the prefill chunks and of the decode tokens of the
    mixed batch (configuration 5), in batch order."""
    kinds = wl.meta["kinds"]
    return ([b for b, k in enumerate(kinds) if k == "prefill"], [b for b, k in enumerate(kinds) if k == "decode"])


# --------------------------------------------------------------------------
# fresh K/V rows for the KV write (recompute-scatter)
# --------------------------------------------------------------------------
@dataclass
class FreshKV:
    segs: np.ndarray       # [n, 4] int32: the workload's fresh segments, descriptor order
    src_rows: np.ndarray   # [n] int32: row of each segment's token 0 in k / v
    k: torch.Tensor        # [rows, H_kv, d] (CPU, workload dtype)
    v: torch.Tensor

    @property
    def rows(self) -> int:
        return int(self.k.shape[0])


def fresh_kv(wl, seed=0, kvscale=0.5):
    """Newly computed K/V rows for every segment of ``wl`` flagged fresh
    (recomputed after eviction, or a chunk's own tokens), laid out as a K/V
    projection writes them: ``[rows, H_kv, d]``, one segment's tokens on
    consecutive rows.  The segments' row ranges follow a random order, so
    source order is not pool order; values are N(0,1) * kvscale rounded to the
    workload dtype (new values, unlike the pool's)."""
    rng = np.random.default_rng(seed)
    fresh = np.ascontiguousarray(wl.segs[(wl.segs[:, 3] & SEG_FRESH) != 0], dtype=np.int32).reshape(-1, 4)
    src_rows = np.zeros(len(fresh), dtype=np.int32)
    row = 0
    for i in rng.permutation(len(fresh)):
        src_rows[i] = row
        row += int(fresh[i, 1])
    shape = (row, wl.num_kv_heads, wl.head_dim)
    k = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(kvscale)).to(wl.torch_dtype)
    v = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(kvscale)).to(wl.torch_dtype)
    return FreshKV(segs=fresh, src_rows=src_rows, k=k, v=v)


# --------------------------------------------------------------------------
# small custom cases (parity edge cases)
# --------------------------------------------------------------------------
def custom(seqs, *, H_q=4, H_kv=2, d=64, dtype="bf16", num_blocks=None, seed=0,
           qscale=0.5, kvscale=0.5, scale=0.0, causal=1, shuffle=True, name="custom"):
    """Build a workload from explicit per-sequence specs.

    ``seqs`` is a list of ``(segments, q_positions)`` where ``segments`` is a
    list of ``(pos_start, len)`` or ``(pos_start, len, flags)`` tuples.
    """
    rng = np.random.default_rng(seed)
    need = sum(-(-s[1] // BLOCK_SIZE) for segs, _ in seqs for s in segs)
    nb = num_blocks if num_blocks is not None else max(2 * need, 4)
    b = _Builder(rng, nb)
    for segs, qp in seqs:
        built = [b.segment(s[0], s[1], s[2] if len(s) > 2 else 0) for s in segs]
        b.add_sequence(built, qp, shuffle=shuffle)
    return b.finish(name, dtype, H_q, H_kv, d, qscale=qscale, kvscale=kvscale, scale=scale, causal=causal)


def random_case(seed, *, batch=3, H_q=8, H_kv=2, d=128, dtype="bf16", max_ctx=300,
                max_chunk=70, decode_frac=0.3, gaps=True, qscale=0.5):
    """Random multi-segment prefill/decode mix with ragged lengths and gaps."""
    rng = np.random.default_rng(seed)
    specs = []
    for _ in range(batch):
        L = int(rng.integers(1, max_ctx, endpoint=True))
        n = int(rng.integers(1, min(L, 8), endpoint=True))
        sizes = _composition(rng, L, n)
        segs, pos = [], int(rng.integers(0, 40))
        for s in sizes:
            segs.append((pos, s, int(rng.random() < 0.25)))
            pos += s + (int(rng.integers(0, 30)) if gaps else 0)
        if rng.random() < decode_frac:
            qp = [segs[-1][0] + segs[-1][1] - 1]
        else:
            c = int(rng.integers(1, max_chunk, endpoint=True))
            segs.append((pos, c, SEG_FRESH))
            qp = list(range(pos, pos + c))
        specs.append((segs, qp))
    return custom(specs, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, seed=seed + 1000,
                  qscale=qscale, name=f"random_{seed}")
