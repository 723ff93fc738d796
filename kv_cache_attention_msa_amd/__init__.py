"""Multi-Segment Attention (MSA) for AMD MI355X (gfx950): Python binding of libmsa.

This module only marshals arguments into the C ABI declared in
``include/msa.h``; every step of the attention runs in the library's HIP
kernels.  PyTorch tensors are accepted for device memory and the current HIP
stream is used by default.  There is no fallback: if ``libmsa.so`` is missing
or fails to load, importing the binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = [
    "MsaError", "Pool", "SegDesc", "forward", "forward_noalloc", "write_kv", "plan_debug", "library_path", "load_library",
    "use_library",
    "LatencyModel", "latency_fit", "chunk_blocks", "EvictIndex", "lambda_from_lifespan",
    "BF16", "FP32", "SEG_FRESH", "BLOCK_SIZE", "EXPORTED_SYMBOLS",
    "KERNEL_PREFILL", "KERNEL_DECODE", "KERNEL_FP32", "KERNEL_MERGE", "KERNEL_UPLOAD", "KERNEL_WRITE",
    "OPT_TIMING", "OPT_SPLIT_BLOCKS", "OPT_NUM_CUS", "OPT_CHECK_BLOCK_IDS", "OPT_PHASE_TRACE", "OPT_CHUNK_WAVES",
]

BF16, FP32 = 0, 1
SEG_FRESH = 1
BLOCK_SIZE = 16
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_OOM, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5
OPT_TIMING, OPT_SPLIT_BLOCKS, OPT_NUM_CUS, OPT_CHECK_BLOCK_IDS, OPT_PHASE_TRACE, OPT_CHUNK_WAVES = 1, 2, 3, 4, 5, 6
KERNEL_PREFILL, KERNEL_DECODE, KERNEL_FP32, KERNEL_MERGE, KERNEL_UPLOAD, KERNEL_WRITE = 0, 1, 2, 3, 4, 5

EXPORTED_SYMBOLS = (
    "msa_create_pool", "msa_pool_kv_ptrs", "msa_destroy_pool", "msa_forward", "msa_forward_noalloc",
    "msa_write_kv", "msa_last_error",
    "msa_pool_set_option", "msa_pool_kernel_time", "msa_pool_kernel_samples", "msa_plan_debug",
    "msa_latency_fit", "msa_latency_eval", "msa_latency_delta_b", "msa_chunk_blocks",
    "msa_evict_create", "msa_evict_destroy", "msa_evict_insert", "msa_evict_touch", "msa_evict_set_position",
    "msa_evict_remove", "msa_evict_pop", "msa_evict_scan_min", "msa_evict_score", "msa_evict_set_lambda",
    "msa_evict_lambda_from_lifespan", "msa_evict_size",
)

_ERR_NAMES = {ERR_INVALID_ARG: "INVALID_ARG", ERR_UNSUPPORTED: "UNSUPPORTED", ERR_OOM: "OOM",
              ERR_WORKSPACE: "WORKSPACE", ERR_HIP: "HIP"}


class MsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"MSA_ERR_{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


# ---- C structures (must match include/msa.h) ---------------------------------
class _PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("device", ctypes.c_int32)]


class _SegDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("q_offsets", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
                ("seg_offsets", ctypes.c_void_p), ("segs", ctypes.c_void_p),
                ("block_table_len", ctypes.c_int32), ("scale", ctypes.c_float),
                ("causal", ctypes.c_int32)]


class _LatencyModel(ctypes.Structure):
    _fields_ = [("k", ctypes.c_double * 5), ("rms", ctypes.c_double), ("n", ctypes.c_int32),
                ("relative", ctypes.c_int32)]


PLAN_ITEM_DTYPE = np.dtype([("kind", "<i4"), ("seq", "<i4"), ("kv_head", "<i4"), ("q_row0", "<i4"),
                            ("n_q", "<i4"), ("blk_begin", "<i4"), ("blk_end", "<i4"), ("part_row", "<i4"),
                            ("launch", "<i4")])
PLAN_BLOCK_DTYPE = np.dtype([("bt_index", "<i4"), ("pos0", "<i4"), ("valid", "<i4")])

_lib = None
_lib_name = "libmsa.so"


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), _lib_name)


def use_library(name: str) -> None:
    """Select the in-tree library file to load (before the first call):
    "libmsa.so" (default) or "libmsa_trace.so", the measurement build whose
    chunk kernel records phase clocks (OPT_PHASE_TRACE)."""
    global _lib_name
    if _lib is not None and name != _lib_name:
        raise RuntimeError(f"{_lib_name} is already loaded")
    if name not in ("libmsa.so", "libmsa_trace.so"):
        raise ValueError(f"unknown library {name!r}")
    _lib_name = name


def load_library():
    """Load libmsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m kv_cache_attention_msa_amd.csrc.build)")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.msa_create_pool.argtypes = [ctypes.POINTER(_PoolDesc), P, P, ctypes.POINTER(P)]
    lib.msa_pool_kv_ptrs.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(P)]
    lib.msa_destroy_pool.argtypes = [P]
    lib.msa_forward.argtypes = [P, ctypes.POINTER(_SegDesc), P, P, P, P, P]
    lib.msa_forward_noalloc.argtypes = [P, ctypes.POINTER(_SegDesc), P, P, P, P, P]
    lib.msa_write_kv.argtypes = [P, P, P, I32, P, P, I32, P, I32, P]
    lib.msa_last_error.argtypes = []
    lib.msa_last_error.restype = ctypes.c_char_p
    lib.msa_pool_set_option.argtypes = [P, I32, I64]
    lib.msa_pool_kernel_time.argtypes = [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64), I32]
    lib.msa_pool_kernel_samples.argtypes = [P, I32, P, I32, ctypes.POINTER(I32)]
    lib.msa_plan_debug.argtypes = [ctypes.POINTER(_SegDesc), I32, I32, I32, I32, I32, P, I32,
                                   ctypes.POINTER(I32), P, I32, ctypes.POINTER(I32)]
    D = ctypes.c_double
    lib.msa_latency_fit.argtypes = [P, I32, I32, ctypes.POINTER(_LatencyModel)]
    lib.msa_latency_eval.argtypes = [ctypes.POINTER(_LatencyModel), D, D, D, D, ctypes.POINTER(D)]
    lib.msa_latency_delta_b.argtypes = [ctypes.POINTER(_LatencyModel), D, D, ctypes.POINTER(D)]
    lib.msa_chunk_blocks.argtypes = [ctypes.POINTER(_LatencyModel), D, D, D, I32, D, ctypes.POINTER(I32)]
    lib.msa_evict_create.argtypes = [ctypes.POINTER(_LatencyModel), D, D, ctypes.POINTER(P)]
    lib.msa_evict_destroy.argtypes = [P]
    lib.msa_evict_insert.argtypes = [P, I64, D, D, D]
    lib.msa_evict_touch.argtypes = [P, I64, D]
    lib.msa_evict_set_position.argtypes = [P, I64, D, D]
    lib.msa_evict_remove.argtypes = [P, I64]
    lib.msa_evict_pop.argtypes = [P, D, ctypes.POINTER(I64), ctypes.POINTER(D)]
    lib.msa_evict_scan_min.argtypes = [P, D, ctypes.POINTER(I64), ctypes.POINTER(D)]
    lib.msa_evict_score.argtypes = [P, I64, D, ctypes.POINTER(D)]
    lib.msa_evict_set_lambda.argtypes = [P, D, D]
    lib.msa_evict_lambda_from_lifespan.argtypes = [D, D, D, D, ctypes.POINTER(D)]
    lib.msa_evict_size.argtypes = [P, ctypes.POINTER(I64)]
    for name in EXPORTED_SYMBOLS:
        if name != "msa_last_error":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != OK:
        raise MsaError(rc, load_library().msa_last_error().decode())


def _ptr(x) -> int:
    """Device/host address of a torch tensor, numpy array, or an int."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return int(x.data_ptr())


def _current_stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else int(stream.cuda_stream)
    import torch
    if torch.cuda.is_available():
        return int(torch.cuda.current_stream().cuda_stream)
    return 0


class SegDesc:
    """Host-side segment descriptors for one msa_forward call (see msa_seg_desc)."""

    def __init__(self, q_offsets, q_pos, seg_offsets, segs, block_table_len, num_q_heads,
                 scale: float = 0.0, causal: bool = True):
        self.q_offsets = np.ascontiguousarray(q_offsets, dtype=np.int32)
        self.q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
        self.seg_offsets = np.ascontiguousarray(seg_offsets, dtype=np.int32)
        self.segs = np.ascontiguousarray(np.asarray(segs, dtype=np.int32).reshape(-1, 4))
        self.total_q = int(self.q_offsets[-1]) if len(self.q_offsets) else 0
        self.num_q_heads = int(num_q_heads)
        self.block_table_len = int(block_table_len)
        self.c = _SegDesc(len(self.q_offsets) - 1, int(num_q_heads),
                          self.q_offsets.ctypes.data, self.q_pos.ctypes.data,
                          self.seg_offsets.ctypes.data, self.segs.ctypes.data,
                          int(block_table_len), float(scale), int(bool(causal)))

    @classmethod
    def from_workload(cls, wl):
        return cls(wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, len(wl.block_table),
                   wl.num_q_heads, wl.scale, bool(wl.causal))


class Pool:
    """A block-paged KV pool: K and V of shape [num_blocks, num_kv_heads, 16, head_dim].

    Pass torch tensors ``k`` and ``v`` to wrap caller memory, or neither to let
    the library allocate the pool.
    """

    def __init__(self, num_blocks, num_kv_heads, head_dim, dtype=BF16, k=None, v=None, device=0):
        lib = load_library()
        if (k is None) != (v is None):
            raise ValueError("give both k and v, or neither")
        if k is not None:
            for t in (k, v):
                if not t.is_contiguous() or tuple(t.shape) != (num_blocks, num_kv_heads, BLOCK_SIZE, head_dim):
                    raise ValueError("k/v must be contiguous [num_blocks, num_kv_heads, 16, head_dim]")
            device = k.device.index or 0
        self._keep = (k, v)
        self.desc = _PoolDesc(num_blocks, BLOCK_SIZE, num_kv_heads, head_dim, dtype, device)
        h = ctypes.c_void_p()
        _check(lib.msa_create_pool(ctypes.byref(self.desc), _ptr(k), _ptr(v), ctypes.byref(h)))
        self.handle = h
        self.num_blocks, self.num_kv_heads, self.head_dim, self.dtype = num_blocks, num_kv_heads, head_dim, dtype

    def kv_ptrs(self):
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        _check(load_library().msa_pool_kv_ptrs(self.handle, ctypes.byref(k), ctypes.byref(v)))
        return k.value, v.value

    def set_option(self, option: int, value: int):
        _check(load_library().msa_pool_set_option(self.handle, option, int(value)))

    def kernel_time(self, kind: int, reset: bool = False):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(load_library().msa_pool_kernel_time(self.handle, kind, ctypes.byref(ms), ctypes.byref(n), int(reset)))
        return ms.value, n.value

    def kernel_samples(self, kind: int, max_samples: int = 1 << 16):
        """Per-launch durations (ms) of `kind` since the last reset, oldest first."""
        out = np.zeros(max_samples, dtype=np.float64)
        n = ctypes.c_int32()
        _check(load_library().msa_pool_kernel_samples(self.handle, kind, out.ctypes.data, max_samples,
                                                      ctypes.byref(n)))
        return out[:n.value]

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _check(load_library().msa_destroy_pool(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def forward(q, seg_desc: SegDesc, block_table, pool: Pool, out, lse=None, stream=None):
    """Enqueue MSA for one batch on ``stream`` (default: torch's current stream).

    ``q``/``out``: [total_q, num_q_heads, head_dim] device tensors of the pool
    dtype (more rows are allowed; rows past total_q are not touched);
    ``block_table``: int32 device tensor; ``lse``: float32 [total_q,
    num_q_heads] device tensor or None.
    """
    _check_forward_tensors(q, seg_desc, block_table, pool, out, lse)
    _check(load_library().msa_forward(_ptr(q), ctypes.byref(seg_desc.c), _ptr(block_table), pool.handle,
                                      _ptr(out), _ptr(lse), _current_stream(stream)))


def forward_noalloc(q, seg_desc: SegDesc, block_table, pool: Pool, out, lse=None, stream=None):
    """As ``forward``, through msa_forward_noalloc: the call allocates no device
    memory (its plan and split partials live in the library's fixed per-GPU
    scratch; calls on one GPU must not overlap)."""
    _check_forward_tensors(q, seg_desc, block_table, pool, out, lse)
    _check(load_library().msa_forward_noalloc(_ptr(q), ctypes.byref(seg_desc.c), _ptr(block_table), pool.handle,
                                              _ptr(out), _ptr(lse), _current_stream(stream)))


def _is_tensor(x) -> bool:
    return hasattr(x, "data_ptr") and hasattr(x, "shape")


def _check_forward_tensors(q, d: SegDesc, block_table, pool: Pool, out, lse):
    """Shape, dtype and layout checks of the torch tensors handed to msa_forward
    (the C ABI receives bare pointers and cannot check sizes).  Raw integer
    addresses are passed through unchecked."""
    if d.total_q == 0:
        return
    # Row counts may exceed total_q (buffers sized for a larger batch).
    rows, inner = d.total_q, (d.num_q_heads, pool.head_dim)
    elt = 4 if pool.dtype == FP32 else 2
    for name, t in (("q", q), ("out", out)):
        if _is_tensor(t):
            if (t.dim() != 3 or t.shape[0] < rows or tuple(t.shape[1:]) != inner or not t.is_contiguous()
                    or t.element_size() != elt or not t.is_cuda):
                raise ValueError(f"{name} must be a contiguous device tensor [>= {rows}, {inner[0]}, {inner[1]}] "
                                 "of the pool dtype")
    if _is_tensor(lse):
        if (lse.dim() != 2 or lse.shape[0] < rows or lse.shape[1] != inner[0] or not lse.is_contiguous()
                or lse.element_size() != 4 or not lse.dtype.is_floating_point or not lse.is_cuda):
            raise ValueError(f"lse must be a contiguous float32 device tensor [>= {rows}, {inner[0]}]")
    if _is_tensor(block_table):
        if (block_table.element_size() != 4 or block_table.dtype.is_floating_point or not block_table.is_cuda
                or not block_table.is_contiguous() or block_table.numel() < d.block_table_len):
            raise ValueError("block_table must be a contiguous int32 device tensor of at least "
                             f"block_table_len = {d.block_table_len} entries")


def write_kv(pool: Pool, k_src, v_src, segs, src_rows, block_table, stream=None):
    """Enqueue the KV write of fresh rows into the pool (see msa_write_kv).

    ``k_src``/``v_src``: contiguous [rows, num_kv_heads, head_dim] device
    tensors of the pool dtype; ``segs``: int32 [n, 4] (pos_start, len,
    bt_start, flags); ``src_rows``: int32 [n], row of each segment's token 0;
    ``block_table``: int32 device tensor.
    """
    segs = np.ascontiguousarray(np.asarray(segs, dtype=np.int32).reshape(-1, 4))
    src_rows = np.ascontiguousarray(src_rows, dtype=np.int32).reshape(-1)
    if len(src_rows) != len(segs):
        raise ValueError("segs and src_rows differ in length")
    rows = 0
    for t in (k_src, v_src):
        if t is None:
            continue
        if not t.is_contiguous() or t.dim() != 3 or tuple(t.shape[1:]) != (pool.num_kv_heads, pool.head_dim):
            raise ValueError("k_src/v_src must be contiguous [rows, num_kv_heads, head_dim]")
        if t.element_size() != (4 if pool.dtype == FP32 else 2):
            raise ValueError("k_src/v_src element type differs from the pool's")
        rows = t.shape[0]
    if k_src is not None and v_src is not None and k_src.shape != v_src.shape:
        raise ValueError("k_src and v_src differ in shape")
    _check(load_library().msa_write_kv(pool.handle, _ptr(k_src), _ptr(v_src), int(rows), segs.ctypes.data,
                                       src_rows.ctypes.data, len(segs), _ptr(block_table),
                                       int(block_table.shape[0]) if block_table is not None else 0,
                                       _current_stream(stream)))


class LatencyModel:
    """A fitted Eq. 5 latency model (see include/msa_latency.h); sizes in blocks."""

    def __init__(self, c: _LatencyModel):
        self.c = c

    @classmethod
    def from_coefficients(cls, k):
        """A model with given k1..k5 (no fit)."""
        c = _LatencyModel()
        for i, v in enumerate(k):
            c.k[i] = float(v)
        return cls(c)

    @property
    def k(self):
        return list(self.c.k)

    @property
    def rms(self) -> float:
        return self.c.rms

    def __call__(self, l1, q1, l2, q2) -> float:
        t = ctypes.c_double()
        _check(load_library().msa_latency_eval(ctypes.byref(self.c), l1, q1, l2, q2, ctypes.byref(t)))
        return t.value

    def delta_b(self, l1, q1) -> float:
        t = ctypes.c_double()
        _check(load_library().msa_latency_delta_b(ctypes.byref(self.c), l1, q1, ctypes.byref(t)))
        return t.value


def latency_fit(samples, relative: bool = True) -> LatencyModel:
    """Fit k1..k5 to rows (l1, q1, l2, q2, T) (host only)."""
    s = np.ascontiguousarray(np.asarray(samples, dtype=np.float64).reshape(-1, 5))
    m = _LatencyModel()
    _check(load_library().msa_latency_fit(s.ctypes.data, len(s), int(bool(relative)), ctypes.byref(m)))
    return LatencyModel(m)


def chunk_blocks(model: LatencyModel, l1, q1, l2, remaining: int, budget: float) -> int:
    """Blocks to prefill in the next step under a step-time budget (see msa_chunk_blocks)."""
    c = ctypes.c_int32()
    _check(load_library().msa_chunk_blocks(ctypes.byref(model.c), l1, q1, l2, int(remaining), budget,
                                           ctypes.byref(c)))
    return c.value


class EvictIndex:
    """Eviction order of cached KV blocks (see include/msa_evict.h): the block of
    lowest score c * n * min(1, lambda * exp(-x / s)) is evicted first, with c
    the Eq. 5 recomputation cost from ``model``."""

    def __init__(self, model: LatencyModel, s: float, lam: float):
        h = ctypes.c_void_p()
        _check(load_library().msa_evict_create(ctypes.byref(model.c), float(s), float(lam), ctypes.byref(h)))
        self.handle = h

    def insert(self, block: int, l1: float, q1: float, now: float):
        _check(load_library().msa_evict_insert(self.handle, int(block), float(l1), float(q1), float(now)))

    def touch(self, block: int, now: float):
        _check(load_library().msa_evict_touch(self.handle, int(block), float(now)))

    def set_position(self, block: int, l1: float, q1: float):
        _check(load_library().msa_evict_set_position(self.handle, int(block), float(l1), float(q1)))

    def remove(self, block: int):
        _check(load_library().msa_evict_remove(self.handle, int(block)))

    def _pick(self, fn, now):
        b, sc = ctypes.c_int64(), ctypes.c_double()
        _check(fn(self.handle, float(now), ctypes.byref(b), ctypes.byref(sc)))
        return b.value, sc.value

    def pop(self, now: float):
        """Evict: (block, score) of the lowest score at ``now``."""
        return self._pick(load_library().msa_evict_pop, now)

    def scan_min(self, now: float):
        """(block, score) that pop would take, by rescoring every block (O(n))."""
        return self._pick(load_library().msa_evict_scan_min, now)

    def score(self, block: int, now: float) -> float:
        sc = ctypes.c_double()
        _check(load_library().msa_evict_score(self.handle, int(block), float(now), ctypes.byref(sc)))
        return sc.value

    def set_lambda(self, lam: float, now: float):
        _check(load_library().msa_evict_set_lambda(self.handle, float(lam), float(now)))

    def __len__(self):
        n = ctypes.c_int64()
        _check(load_library().msa_evict_size(self.handle, ctypes.byref(n)))
        return n.value

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            load_library().msa_evict_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lambda_from_lifespan(tau: float, tau0: float, alpha: float, beta: float) -> float:
    """Eq. 10: lambda = exp((tau - tau0) / beta - tau / alpha)."""
    lam = ctypes.c_double()
    _check(load_library().msa_evict_lambda_from_lifespan(float(tau), float(tau0), float(alpha), float(beta),
                                                          ctypes.byref(lam)))
    return lam.value


def plan_debug(seg_desc: SegDesc, num_kv_heads: int, head_dim: int, dtype: int = BF16,
               num_cus: int = 256, split_blocks: int = 0):
    """Run the host planner alone; returns (items, blocks) as numpy structured arrays."""
    lib = load_library()
    ni, nb = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.msa_plan_debug(ctypes.byref(seg_desc.c), num_kv_heads, head_dim, dtype, num_cus, split_blocks,
                              None, 0, ctypes.byref(ni), None, 0, ctypes.byref(nb)))
    items = np.zeros(ni.value, dtype=PLAN_ITEM_DTYPE)
    blocks = np.zeros(nb.value, dtype=PLAN_BLOCK_DTYPE)
    _check(lib.msa_plan_debug(ctypes.byref(seg_desc.c), num_kv_heads, head_dim, dtype, num_cus, split_blocks,
                              items.ctypes.data, len(items), ctypes.byref(ni),
                              blocks.ctypes.data, len(blocks), ctypes.byref(nb)))
    return items, blocks
