"""msa_forward_noalloc: the attention entry point that allocates no device memory.

GPU: called through the C ABI (ctypes, no binding checks in between) three
times in a row -- the full-size 64-sequence decode workload (split tiles, so
the merge reads partials from the fixed scratch), then a smaller batch with
forced KV splits, then a small batch of prefill chunks and decode tokens (one
fused launch, forced splits on both kinds) -- each compared bit for bit with
msa_forward on the same pool and inputs, and element-wise with the fp64
oracle.
CPU: a call whose plan exceeds the fixed scratch is refused before any HIP
call.
"""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_attention_msa_amd as msa
import workloads as W
from msa_gpu_util import GpuCase, compare, oracle_result


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _noalloc_raw(case):
    """msa_forward_noalloc straight through the C ABI on torch's current stream."""
    lib = msa.load_library()
    stream = int(torch.cuda.current_stream().cuda_stream)
    return lib.msa_forward_noalloc(case.q.data_ptr(), ctypes.byref(case.desc.c), case.bt.data_ptr(),
                                   case.pool.handle, case.out.data_ptr(), case.lse.data_ptr(), stream)


def _run_pair(wl, split_blocks):
    print(f"[noalloc] {wl.name} split_blocks={split_blocks}", flush=True)
    case = GpuCase(wl)
    try:
        ref_out, ref_lse = case.run(split_blocks)          # msa_forward
        case.out.fill_(float("nan"))
        case.lse.fill_(float("nan"))
        rc = _noalloc_raw(case)
        assert rc == 0, msa.load_library().msa_last_error().decode()
        torch.cuda.synchronize()
        out, lse = case.out.cpu(), case.lse.cpu()
    finally:
        case.close()
    assert torch.equal(_bits(out), _bits(ref_out)), "out differs from msa_forward"
    assert torch.equal(_bits(lse), _bits(ref_lse)), "lse differs from msa_forward"
    o_ref, l_ref = oracle_result(wl)
    compare(wl, out, lse, o_ref, l_ref)


@pytest.mark.gpu
def test_noalloc_matches_forward_twice_second_smaller():
    big = W.config3()
    small = W.random_case(81, batch=2, H_q=8, H_kv=2, d=128, max_ctx=500, max_chunk=60)
    mixed = W.custom([([(0, 256), (300, 64)], list(range(300, 364))), ([(0, 200)], [199]), ([(16, 500)], [515]),
                      ([(0, 90), (120, 33)], [152])], H_q=8, H_kv=2, d=128, seed=83, name="mixed_small")
    _run_pair(big, split_blocks=0)       # automatic splits: decode partials + merge in the scratch
    _run_pair(small, split_blocks=3)     # forced splits on chunk items
    _run_pair(mixed, split_blocks=3)     # decode items inside the chunk launch, both kinds split


def test_noalloc_refuses_plans_beyond_the_scratch():
    """300 000 KV blocks need 2.4 MB of block list, more than the scratch's
    2 MiB plan area: refused with MSA_ERR_WORKSPACE before any HIP call (the
    pool wraps caller pointers, so no HIP call is made at all)."""
    lib = msa.load_library()
    nblk = 300_000
    desc = msa._PoolDesc(nblk, 16, 1, 64, msa.BF16, 0)
    h = ctypes.c_void_p()
    assert lib.msa_create_pool(ctypes.byref(desc), 0x10000, 0x20000, ctypes.byref(h)) == 0
    try:
        d = msa.SegDesc([0, 1], [16 * nblk - 1], [0, 1], np.array([[0, 16 * nblk, 0, 0]]), nblk, 1)
        rc = lib.msa_forward_noalloc(0x1000, ctypes.byref(d.c), 0x2000, h, 0x3000, 0x4000, 0)
        assert rc == msa.ERR_WORKSPACE
        assert "fixed scratch" in lib.msa_last_error().decode()
    finally:
        lib.msa_destroy_pool(h)
