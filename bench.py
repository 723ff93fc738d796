"""Benchmark Multi-Segment Attention (libmsa) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline] [--no-secondary]

One step is one msa_forward call over the whole workload: host planning, the
plan upload and every kernel (chunk/prefill, decode, merge), with q, the K/V
pool and the block table already resident in HBM.  The headline workload is
chunked prefill (4 sequences, GQA 32/8, head_dim 128, 4096-token context in 6
scattered segments plus a 512-token chunk), reported in TFLOP/s of visible
(query, key) pairs.  Reported alongside, each against its roofline:
  * decode (64 sequences, 1k-8k-token contexts in 2-16 segments over a
    2M-token pool), HBM GB/s;
  * heavy fragmentation (2 sequences, 32 768-token contexts in 64 segments
    with position gaps, 2048-token chunks), TFLOP/s;
  * the mixed batch (16 sequences, GQA 64/8: 8 prefill chunks and 8 decode
    tokens over 2k-16k-token contexts), whole batch as T_roof / T, and its
    prefill-only and decode-only parts separately;
  * the tiny fp32 case (time only);
  * the KV write (msa_write_kv) of the mixed batch's fresh rows (61 fresh
    segments, 44 820 rows of 8 kv heads x 128) into its 65 536-block pool.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time


def _blas_threads() -> int:
    """Threads for the CPU baseline's BLAS: the CPUs this process may run on,
    capped by an OMP_NUM_THREADS the environment already sets.  Set before
    numpy is first imported, so that OpenBLAS/MKL/OpenMP pick it up."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, str(n))
    return n


BLAS_THREADS = _blas_threads()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA attention TFLOP/s (prefill) and HBM GB/s (decode) vs MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# the device sources each kernel is built from (a traffic record holds only while they are unchanged)
KERNEL_SOURCES = {"prefill": ("kv_cache_attention_msa_amd/csrc/msa_prefill.hip",
                              "kv_cache_attention_msa_amd/csrc/msa_decode_item.h"),
                  "decode": ("kv_cache_attention_msa_amd/csrc/msa_decode.hip",
                             "kv_cache_attention_msa_amd/csrc/msa_decode_item.h"),
                  "write": ("kv_cache_attention_msa_amd/csrc/msa_write.hip",)}
GATE_MFMA, GATE_HBM = 0.60, 0.70     # roofline fractions the benchmark definition asks for


def visible_counts(wl):
    """Per query row: number of keys it sees (k_pos <= q_pos when causal)."""
    import numpy as np
    counts = np.zeros(wl.total_q, dtype=np.int64)
    seq_tokens = np.zeros(wl.batch, dtype=np.int64)
    for b in range(wl.batch):
        segs = wl.segs[wl.seg_offsets[b]:wl.seg_offsets[b + 1]]
        starts, lens = segs[:, 0].astype(np.int64), segs[:, 1].astype(np.int64)
        r = slice(wl.q_offsets[b], wl.q_offsets[b + 1])
        qp = wl.q_pos[r].astype(np.int64)
        if wl.causal:
            c = np.clip(qp[:, None] - starts[None, :] + 1, 0, lens[None, :]).sum(axis=1)
            seq_tokens[b] = int(np.clip(qp.max() - starts + 1, 0, lens).sum()) if len(qp) else 0
        else:
            c = np.full(len(qp), lens.sum())
            seq_tokens[b] = lens.sum() if len(qp) else 0
        counts[r] = c
    return counts, seq_tokens


def work_of(wl):
    """Algorithmic FLOPs and HBM bytes of one MSA call."""
    counts, seq_tokens = visible_counts(wl)
    d, Hq, Hkv = wl.head_dim, wl.num_q_heads, wl.num_kv_heads
    elt = 4 if wl.dtype == "fp32" else 2
    flops = float(counts.sum()) * Hq * 4 * d
    kv_bytes = float(seq_tokens.sum()) * Hkv * d * 2 * elt
    io_bytes = wl.total_q * Hq * d * elt * 2 + wl.total_q * Hq * 4 + len(wl.block_table) * 4
    return flops, kv_bytes + io_bytes


def source_sha(rels):
    """sha256[:16] over the given source files, concatenated in order."""
    h = hashlib.sha256()
    for rel in rels:
        p = os.path.join(ROOT, rel)
        if not os.path.exists(p):
            return None
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_path(kernel, units):
    return os.path.join(ROOT, "profiles", f"{kernel}_traffic_{units}.json")


def traffic_for(kernel, units):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if the
    kernel source still matches the one the counters were taken on."""
    path = traffic_path(kernel, units)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_src_sha") != source_sha(KERNEL_SOURCES[kernel]) or rec.get("units") != units:
        return None
    return rec.get("bytes_per_launch")


def percentiles(samples_ms):
    """p10 / median / p90 of per-launch durations (ms)."""
    import numpy as np
    if len(samples_ms) == 0:
        return None
    p10, p50, p90 = np.percentile(np.asarray(samples_ms), [10, 50, 90])
    return {"p10": float(p10), "p50": float(p50), "p90": float(p90), "n": int(len(samples_ms))}


SETTLE_S = 0.3   # seconds of back-to-back calls before the warm-up steps


def settle(call, seconds=SETTLE_S):
    """Run `call` back to back until the GPU has been busy for `seconds`.

    From idle the GPU needs some tens of milliseconds of load before its clocks
    settle; without this the first timed calls of a short run come out ~12 %
    slower than steady state (0.165 against 0.146 ms per prefill call).  The
    timed region still holds exactly the requested steps."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            call()
        torch.cuda.synchronize()


def run_workload(wl, steps, warmup, kind, cold=False, pool_kv=None):
    """Time msa_forward over the workload: wall clock per call over back-to-back
    calls, then per-kernel HIP-event times (totals and per-launch samples for
    `kind`); with cold, also `kind`'s launch times when a 1 GiB read between
    calls has evicted the Infinity Cache.  pool_kv: resident (K, V) to reuse."""
    import torch
    import kv_cache_attention_msa_amd as msa

    K, V = pool_kv if pool_kv is not None else wl.dense_pool("cuda")
    dt = msa.FP32 if wl.dtype == "fp32" else msa.BF16
    pool = msa.Pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, dt, k=K, v=V)
    q = wl.q.cuda()
    out = torch.empty_like(q)
    lse = torch.empty(wl.total_q, wl.num_q_heads, dtype=torch.float32, device="cuda")
    bt = torch.from_numpy(wl.block_table).cuda()
    desc = msa.SegDesc.from_workload(wl)
    stream = torch.cuda.current_stream()
    settle(lambda: msa.forward(q, desc, bt, pool, out, lse, stream))
    for _ in range(warmup):
        msa.forward(q, desc, bt, pool, out, lse, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        msa.forward(q, desc, bt, pool, out, lse, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel-only timing: HIP events recorded by libmsa around each launch
    pool.set_option(msa.OPT_TIMING, 1)
    pool.kernel_time(kind, reset=True)
    for _ in range(steps):
        msa.forward(q, desc, bt, pool, out, lse, stream)
    torch.cuda.synchronize()
    times = {k: pool.kernel_time(k) for k in (msa.KERNEL_PREFILL, msa.KERNEL_DECODE, msa.KERNEL_FP32,
                                              msa.KERNEL_MERGE, msa.KERNEL_UPLOAD)}
    times["dist"] = percentiles(pool.kernel_samples(kind))
    if cold:
        flush = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
        pool.kernel_time(kind, reset=True)
        for _ in range(steps):
            flush.sum()
            msa.forward(q, desc, bt, pool, out, lse, stream)
        torch.cuda.synchronize()
        times["cold_dist"] = percentiles(pool.kernel_samples(kind))
        del flush
    # host cost of one call (binding checks, planning, packing into the
    # staging ring, enqueueing the kernels) with the GPU idle, so that the call
    # never waits for a staging buffer: median of 9
    pool.set_option(msa.OPT_TIMING, 0)
    host = []
    for _ in range(9):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        msa.forward(q, desc, bt, pool, out, lse, stream)
        host.append(time.perf_counter() - t1)
    torch.cuda.synchronize()
    plan_ms = sorted(host)[len(host) // 2] * 1e3
    pool.close()
    del K, V
    if pool_kv is None:
        torch.cuda.empty_cache()
    return wall / steps * 1e3, times, plan_ms


def run_write(wl, fresh, steps, warmup, pool_kv=None):
    """Time msa_write_kv of the workload's fresh rows into its pool.

    Returns (wall ms per call, warm kernel ms, cold kernel ms, launches): wall
    clock over back-to-back calls; kernel time from HIP events on the launch
    stream, warm (back to back: the 184 MB source can stay in the 256 MB
    Infinity Cache) and cold (a 1 GiB read between calls fills the cache with
    other, clean lines, so the source comes from HBM)."""
    import torch
    import kv_cache_attention_msa_amd as msa

    K, V = pool_kv if pool_kv is not None else wl.dense_pool("cuda")
    pool = msa.Pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, msa.BF16, k=K, v=V)
    ks, vs = fresh.k.cuda(), fresh.v.cuda()
    bt = torch.from_numpy(wl.block_table).cuda()
    flush = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    settle(lambda: msa.write_kv(pool, ks, vs, fresh.segs, fresh.src_rows, bt, stream))
    for _ in range(warmup):
        msa.write_kv(pool, ks, vs, fresh.segs, fresh.src_rows, bt, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        msa.write_kv(pool, ks, vs, fresh.segs, fresh.src_rows, bt, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pool.set_option(msa.OPT_TIMING, 1)
    pool.kernel_time(msa.KERNEL_WRITE, reset=True)
    for _ in range(steps):
        msa.write_kv(pool, ks, vs, fresh.segs, fresh.src_rows, bt, stream)
    torch.cuda.synchronize()
    warm_dist = percentiles(pool.kernel_samples(msa.KERNEL_WRITE))
    warm_ms, warm_n = pool.kernel_time(msa.KERNEL_WRITE, reset=True)
    for _ in range(steps):
        flush.sum()
        msa.write_kv(pool, ks, vs, fresh.segs, fresh.src_rows, bt, stream)
    torch.cuda.synchronize()
    cold_ms, cold_n = pool.kernel_time(msa.KERNEL_WRITE)
    cold_dist = percentiles(pool.kernel_samples(msa.KERNEL_WRITE))
    pool.close()
    del K, V, flush
    torch.cuda.empty_cache()
    run_write.dists = {"warm": warm_dist, "cold": cold_dist}
    return wall / steps * 1e3, warm_ms / max(warm_n, 1), cold_ms / max(cold_n, 1), cold_n


def write_bytes(wl, fresh):
    """Algorithmic bytes of one KV write: every fresh K and V row read once and
    written once, plus one block id per destination block."""
    import numpy as np
    elt = 4 if wl.dtype == "fp32" else 2
    blocks = int(np.sum(-(-fresh.segs[:, 1] // 16))) if len(fresh.segs) else 0
    return 2.0 * 2.0 * fresh.rows * wl.num_kv_heads * wl.head_dim * elt + 4.0 * blocks


def attainable_peaks():
    """What this GPU sustains, measured by the probes of libmsa_peaks.so: a
    streaming HBM read (4 GiB, 16 B per lane) and back-to-back bf16 MFMAs."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_attention_msa_amd", "libmsa_peaks.so"))
    lib.msa_peak_hbm_read.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.msa_peak_hbm_copy.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.msa_peak_hbm_gather.argtypes = [ctypes.c_int32, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.msa_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    gbps, copy, gather, tflops = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    assert lib.msa_peak_hbm_read(4 << 30, 5, ctypes.byref(gbps)) == 0
    assert lib.msa_peak_hbm_copy(1 << 30, 5, ctypes.byref(copy)) == 0
    assert lib.msa_peak_hbm_gather(1 << 18, 5, ctypes.byref(gather)) == 0
    assert lib.msa_peak_mfma_bf16(4000, ctypes.byref(tflops)) == 0
    return {"hbm_read_GBps": gbps.value, "hbm_gather_4KiB_GBps": gather.value, "hbm_copy_GBps": copy.value,
            "mfma_bf16_TFLOPs": tflops.value,
            "how": "libmsa_peaks.so: streaming 4 GiB read; 1 GiB of scattered 4 KiB blocks (of a 2 GiB buffer); "
                   "1 GiB device copy (read + write bytes); v_mfma_f32_32x32x16_bf16 loop on independent accumulators"}


def cpu_baseline(wl, flops_per_row, budget_s=12.0):
    """The fp64 oracle on a bounded sample: whole sequences, taken in order,
    until about budget_s of CPU time has been spent."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import attend
    Kp, Vp = wl.sparse_pools_f64()
    q64 = wl.q_f64()
    done_rows, done_flops, t = 0, 0.0, 0.0
    seqs = 0
    for b in range(wl.batch):
        r0, r1 = int(wl.q_offsets[b]), int(wl.q_offsets[b + 1])
        t0 = time.perf_counter()
        attend(q64, wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, wl.block_table, Kp, Vp,
               wl.num_kv_heads, scale=wl.scale, causal=bool(wl.causal), rows=np.arange(r0, r1))
        t += time.perf_counter() - t0
        done_rows += r1 - r0
        done_flops += float(flops_per_row[r0:r1].sum())
        seqs += 1
        if t >= budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": done_flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{seqs} of {wl.batch} sequences of {wl.name} ({done_rows} query rows x {wl.num_q_heads} "
                      f"heads, all their visible keys), fp64 numpy, {t:.1f} s",
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads_requested": BLAS_THREADS}


def cpu_oracle_configs(budget_s=6.0, row_block=256):
    """The fp64 oracle beside the other benchmark workloads (decode, heavy
    fragmentation, mixed batch), each on a bounded sample: query rows in
    order, in blocks of at most row_block rows of one sequence, until about
    budget_s of CPU time.  Rates in each workload's own unit: GB/s of
    algorithmic bytes for decode (whole sequences of one token), TFLOP/s of
    algorithmic FLOPs otherwise.  Context only."""
    import numpy as np
    import workloads as W
    from oracle import attend
    out = {}
    for wl, unit in ((W.config3(), "GB/s"), (W.config4(), "TFLOP/s"), (W.config5(), "TFLOP/s")):
        Kp, Vp = wl.sparse_pools_f64()
        q64 = wl.q_f64()
        counts, _ = visible_counts(wl)
        t, rows_done, flops, seqs = 0.0, 0, 0.0, []
        for b in range(wl.batch):
            r0, r1 = int(wl.q_offsets[b]), int(wl.q_offsets[b + 1])
            for c0 in range(r0, r1, row_block):
                rows = np.arange(c0, min(r1, c0 + row_block))
                t0 = time.perf_counter()
                attend(q64, wl.q_offsets, wl.q_pos, wl.seg_offsets, wl.segs, wl.block_table, Kp, Vp,
                       wl.num_kv_heads, scale=wl.scale, causal=bool(wl.causal), rows=rows)
                t += time.perf_counter() - t0
                rows_done += len(rows)
                flops += float(counts[rows].sum()) * wl.num_q_heads * 4 * wl.head_dim
                if t >= budget_s:
                    break
            seqs.append(b)
            if t >= budget_s:
                break
        if unit == "GB/s":
            _, nb = work_of(W.subset(wl, seqs, wl.name + "_sample"))
            value = nb / t / 1e9
        else:
            value = flops / t / 1e12
        out[wl.name] = {"value": value, "unit": unit,
                        "sample": f"{rows_done} query rows of the first {len(seqs)} of {wl.batch} sequences "
                                  f"(all heads, all visible keys), fp64 numpy, {t:.1f} s"}
        del Kp, Vp, q64
    return out


# ---------------------------------------------------------------------------
# profiler helpers
# ---------------------------------------------------------------------------
def copy_kernel_run(nbytes, reps=5):
    """A plain device copy of nbytes (one read and one write of each byte),
    used to calibrate the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def _csv_rows(path):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*.csv"), recursive=True) if os.path.isdir(path) else [path]
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(list(csv.DictReader(fh)))
    return rows


def _counter_kib(path, counter, name_part):
    vals = [float(r["Counter_Value"]) for r in _csv_rows(path)
            if r.get("Counter_Name") == counter and name_part in r.get("Kernel_Name", "")]
    return sum(vals) / len(vals) if vals else None, len(vals)


def write_report(args):
    """Turn rocprofv3 output into a short committed summary (and a traffic record)."""
    stats = [r for r in _csv_rows(args.stats) if "AverageNs" in r and r.get("Name") != "KERNEL_DISPATCH"]
    lines = [f"# {args.kernel} on {args.units}", "", "Commands (run from the repository root on an MI355X):", ""]
    for c in args.command:
        lines.append(f"    {c}")
    lines += ["", "## rocprofv3 --kernel-trace --stats", "",
              "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:8]:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    rec = None
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        f_kib, nf = _counter_kib(args.fetch, "FETCH_SIZE", args.kernel)
        w_kib, nw = _counter_kib(args.write, "WRITE_SIZE", args.kernel)
        cf_kib, _ = _counter_kib(args.copy_fetch, "FETCH_SIZE", args.copy_kernel)
        cw_kib, _ = _counter_kib(args.copy_write, "WRITE_SIZE", args.copy_kernel)
        kf = args.copy_bytes / (cf_kib * 1024.0)
        kw = args.copy_bytes / (cw_kib * 1024.0)
        fetch_b, write_b = f_kib * 1024.0 * kf, w_kib * 1024.0 * kw
        rec = {"kernel": args.kernel, "units": args.units, "kernel_src_sha": source_sha(KERNEL_SOURCES[args.key]),
               "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
               "bytes_per_launch": fetch_b + write_b, "fetch_factor": kf, "write_factor": kw,
               "raw_fetch_kib": f_kib, "raw_write_kib": w_kib, "dispatches": [nf, nw]}
        lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
                  f"- kernel: FETCH_SIZE {f_kib:.0f} KiB, WRITE_SIZE {w_kib:.0f} KiB per dispatch "
                  f"(mean of {nf} / {nw} dispatches)",
                  f"- plain copy of {args.copy_bytes} bytes: FETCH_SIZE {cf_kib:.0f} KiB, WRITE_SIZE {cw_kib:.0f} KiB "
                  f"-> scale factors {kf:.3f} (fetch), {kw:.3f} (write)",
                  f"- scaled traffic per launch: {fetch_b / 1e6:.1f} MB read + {write_b / 1e6:.1f} MB written "
                  f"= {(fetch_b + write_b) / 1e6:.1f} MB",
                  f"- kernel sources ({', '.join(os.path.basename(r) for r in KERNEL_SOURCES[args.key])}) "
                  f"sha256[:16]: {rec['kernel_src_sha']}"]
        with open(traffic_path(args.key, args.units), "w") as fh:
            json.dump(rec, fh, indent=1)
    if args.notes:
        lines += ["", "## Notes", ""] + [f"- {n}" for n in args.notes]
    with open(args.report, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {args.report}" + (" and traffic record" if rec else ""))


def latency_model_run(args):
    """Calibrate the Eq. 5 latency model on this GPU and check its dT_B against
    directly measured differences T(l1, q1 + D, l2 - D, q2) - T(l1, q1, l2, q2)."""
    import numpy as np
    from kv_cache_attention_msa_amd import calibrate as C

    D = 16
    bases = [(128, 8, 128, 8), (256, 32, 64, 8), (64, 0, 256, 32), (0, 16, 128, 1), (256, 8, 256, 1)]
    pairs = [p for b in bases for p in (b, (b[0], b[1] + D, b[2] - D, b[3]))]
    t0 = time.perf_counter()
    B = args.latency_batch
    grid = C.measure_grid(batch=B, reps=15, warmup=3, seed=1)
    check = C.measure_grid(grid={"l1": (), "q1": (), "l2": (), "q2": ()}, batch=B, reps=41, warmup=5, seed=2,
                           extra_points=pairs)
    model = C.calibrate(grid)
    rows = []
    for i, b in enumerate(bases):
        t_base, t_moved = check[2 * i, 4], check[2 * i + 1, 4]
        predicted = sum(model.delta_b(b[0], b[1] + j) for j in range(D))
        rows.append({"l1": b[0], "q1": b[1], "l2": b[2], "q2": b[3], "T_us": t_base, "T_moved_us": t_moved,
                     "measured_dT_us": t_moved - t_base, "eq5_dT_us": predicted,
                     "model_T_us": model(*b)})
    # adaptive chunk rule: chunk chosen from the model for a step-time budget, then timed
    import kv_cache_attention_msa_amd as msa
    chunk_cases = [(l1, q1, l2, budget) for (l1, q1, l2) in ((256, 0, 0), (128, 16, 128), (64, 32, 256))
                   for budget in (250.0, 500.0, 1000.0)]
    chosen = [(l1, q1, l2, msa.chunk_blocks(model, l1, q1, l2, 512, budget)) for l1, q1, l2, budget in chunk_cases]
    timed = C.measure_grid(grid={"l1": (), "q1": (), "l2": (), "q2": ()}, batch=B, reps=21, warmup=3, seed=4,
                           extra_points=chosen)
    chunks = [{"l1": c[0], "q1": c[1], "l2": c[2], "budget_us": c[3], "chunk_blocks": p[3], "T_us": t[4]}
              for c, p, t in zip(chunk_cases, chosen, timed)]
    res = {"model": "T = k1 + k2 (q1+q2) + k3 (l1+l2) + k4 q2 (l1+q1+l2+q2) + k5 q1 (l1+q1), sizes in 16-token blocks, T in us",
           "workload": f"{B} requests, GQA 32/8, d 128, bf16; step = msa_write_kv of the q1+q2 fresh blocks + msa_forward "
                       "of their query rows; median of 15 (grid) / 41 (checks) HIP-event timed steps",
           "k": model.k, "rms_rel": model.rms, "n": int(len(grid)), "dT_check_blocks_moved": D, "checks": rows,
           "chunk_rule": chunks,
           "grid": grid.tolist(), "seconds": time.perf_counter() - t0}
    print(json.dumps({k: v for k, v in res.items() if k != "grid"}), flush=True)
    if args.latency_out:
        with open(args.latency_out, "w") as fh:
            json.dump(res, fh)


def latency_report(src, dst, command):
    """Short text summary of a latency-model run (no GPU needed)."""
    res = json.load(open(src))
    k = res["k"]
    lines = ["# Eq. 5 latency model on one MI355X", "", "Commands (run from the repository root on an MI355X):", "",
             f"    {command}",
             f"    python bench.py --latency-report {src} --report {dst}", "",
             f"Model: {res['model']}.", "", f"Workload: {res['workload']}.", "",
             "## Fitted coefficients (least squares, residuals relative to T)", "",
             "| k1 (us) | k2 (us/block) | k3 (us/block) | k4 (us/block^2) | k5 (us/block^2) | rms rel. residual | samples |",
             "|---|---|---|---|---|---|---|",
             f"| {k[0]:.3f} | {k[1]:.4f} | {k[2]:.5f} | {k[3]:.3e} | {k[4]:.3e} | {res['rms_rel']:.3f} | {res['n']} |",
             "", f"## dT_B: moving {res['dT_check_blocks_moved']} blocks from l2 to q1", "",
             "| l1 | q1 | l2 | q2 | T measured (us) | T model (us) | dT measured (us) | dT from Eq. 5 (us) |",
             "|---|---|---|---|---|---|---|---|"]
    for r in res["checks"]:
        lines.append(f"| {r['l1']} | {r['q1']} | {r['l2']} | {r['q2']} | {r['T_us']:.1f} | {r['model_T_us']:.1f} | "
                     f"{r['measured_dT_us']:.1f} | {r['eq5_dT_us']:.1f} |")
    if res.get("chunk_rule"):
        lines += ["", "## Adaptive chunk size: largest chunk whose modelled step time fits the budget (512 blocks left)", "",
                  "| l1 | q1 | l2 | budget (us) | chunk (blocks) | step time measured (us) |", "|---|---|---|---|---|---|"]
        for r in res["chunk_rule"]:
            lines.append(f"| {r['l1']} | {r['q1']} | {r['l2']} | {r['budget_us']:.0f} | {r['chunk_blocks']} | {r['T_us']:.1f} |")
    with open(dst, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {dst}")


def evict_sweep(report=None, sizes=(4000, 5000, 6000, 7000, 8000, 9000, 10000), cycles=2000, seed=0):
    """Eviction time against the number of cached blocks (the comparison of the
    paper's Figure 9): per eviction, the lowest-score block leaves and a new
    one is cached, with two hits on random blocks in between.  Timed: the
    library's O(log n) index (pop + insert), the same index evicting by its
    O(n) rescoring scan (scan_min + remove + insert), the O(n) oracle in
    Python, and an O(1) LRU list (Python OrderedDict) for scale.  Host only."""
    import collections
    import numpy as np
    import kv_cache_attention_msa_amd as msa
    from oracle import EvictOracle
    k = [12.0, 0.4, 0.2, 0.05, 0.06]
    s_decay, lam = 50.0, 4.0
    model = msa.LatencyModel.from_coefficients(k)
    rows = []
    for n in sizes:
        rng = np.random.default_rng(seed + n)
        pos = rng.integers(0, 512, size=(n + cycles, 2)).astype(float)
        hits = rng.integers(0, n, size=(cycles, 2))
        res = {"blocks": n}
        for kind in ("heap", "scan", "oracle", "lru"):
            cyc = cycles if kind != "oracle" else max(20, cycles // 50)
            idx = msa.EvictIndex(model, s_decay, lam) if kind in ("heap", "scan") else None
            o = EvictOracle(k, s_decay, lam) if kind == "oracle" else None
            lru = collections.OrderedDict() if kind == "lru" else None
            live = []
            for b in range(n):
                t = b * 0.01
                if idx is not None:
                    idx.insert(b, pos[b, 0], pos[b, 1], t)
                elif o is not None:
                    o.insert(b, pos[b, 0], pos[b, 1], t)
                else:
                    lru[b] = t
                live.append(b)
            now, spent = n * 0.01, 0.0
            warm = cyc // 10    # untimed first evictions (caches, allocator)
            for c in range(cyc):
                now += 0.01
                for h in hits[c]:
                    b = live[int(h) % len(live)]
                    if idx is not None:
                        idx.touch(b, now)
                    elif o is not None:
                        o.touch(b, now)
                    else:
                        lru.move_to_end(b)
                nb = n + c
                t0 = time.perf_counter()
                if kind == "heap":
                    gone, _ = idx.pop(now)
                    idx.insert(nb, pos[nb, 0], pos[nb, 1], now)
                elif kind == "scan":
                    gone, _ = idx.scan_min(now)
                    idx.remove(gone)
                    idx.insert(nb, pos[nb, 0], pos[nb, 1], now)
                elif kind == "oracle":
                    gone, _ = o.pop(now)
                    o.insert(nb, pos[nb, 0], pos[nb, 1], now)
                else:
                    gone, _ = lru.popitem(last=False)
                    lru[nb] = now
                if c >= warm:
                    spent += time.perf_counter() - t0
                live[live.index(gone)] = nb
            res[kind + "_us"] = spent / (cyc - warm) * 1e6
            if idx is not None:
                idx.close()
        rows.append(res)
        print(json.dumps(res), flush=True)
    if report:
        lines = ["# Eviction time against cached blocks (host CPU)", "",
                 "Command (run from the repository root):", "", "    python bench.py --evict-sweep --report " + report, "",
                 f"Per eviction: the lowest-score block leaves and a new one is cached (two hits on random blocks in "
                 f"between, not timed); score c * n * min(1, lambda exp(-x / s)) with lambda {lam}, s {s_decay}; mean of "
                 f"{cycles} evictions ({max(20, cycles // 50)} for the Python oracle), the first tenth untimed. "
                 f"The library's figures include two (index) or three (scan) Python-to-C calls per eviction, about "
                 f"1 us each, so the O(log n) work itself is a fraction of its column. CPU: {cpu_model()}.", "",
                 "| cached blocks | O(log n) index (us) | O(n) rescoring scan, native (us) | O(n) oracle, Python (us) | O(1) LRU, Python (us) |",
                 "|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| {r['blocks']} | {r['heap_us']:.2f} | {r['scan_us']:.1f} | {r['oracle_us']:.0f} | {r['lru_us']:.2f} |")
        with open(report, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {report}")
    return rows


PHASES = ("QK product issued", "LDS DMA issued", "mask", "softmax", "PV product issued", "metadata + barrier")


def phase_trace_run(args):
    """Per-phase shader clocks of the chunk kernel's steps on the prefill
    workload, from the measurement build libmsa_trace.so (MSA_PHASE_TRACE:
    s_memtime between scheduling fences at every phase boundary, summed per
    work item and wave).  Prints one JSON line; with --report, a summary."""
    import numpy as np
    import torch
    import kv_cache_attention_msa_amd as msa
    import workloads as W
    msa.use_library("libmsa_trace.so")
    wl = W.config2()
    f, _ = work_of(wl)
    K, V = wl.dense_pool("cuda")
    pool = msa.Pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, msa.BF16, k=K, v=V)
    q = wl.q.cuda()
    out = torch.empty_like(q)
    lse = torch.empty(wl.total_q, wl.num_q_heads, dtype=torch.float32, device="cuda")
    bt = torch.from_numpy(wl.block_table).cuda()
    desc = msa.SegDesc.from_workload(wl)
    items, _ = msa.plan_debug(desc, wl.num_kv_heads, wl.head_dim)
    n_items = int((items["launch"] == msa.KERNEL_PREFILL).sum())
    trace = torch.zeros(n_items * 8 * 8, dtype=torch.int64, device="cuda")   # 8 wave slots per item
    stream = torch.cuda.current_stream()
    settle(lambda: msa.forward(q, desc, bt, pool, out, lse, stream))
    pool.set_option(msa.OPT_TIMING, 1)
    pool.kernel_time(msa.KERNEL_PREFILL, reset=True)
    for _ in range(args.steps):
        msa.forward(q, desc, bt, pool, out, lse, stream)
    torch.cuda.synchronize()
    plain_ms, n = pool.kernel_time(msa.KERNEL_PREFILL, reset=True)
    pool.set_option(msa.OPT_PHASE_TRACE, trace.data_ptr())
    sums = np.zeros(8)
    for _ in range(args.steps):
        trace.zero_()
        msa.forward(q, desc, bt, pool, out, lse, stream)
        torch.cuda.synchronize()
        sums += trace.view(-1, 8).cpu().numpy().astype(np.float64).sum(axis=0)
    traced_ms, n2 = pool.kernel_time(msa.KERNEL_PREFILL)
    pool.set_option(msa.OPT_PHASE_TRACE, 0)
    pool.close()
    steps = sums[0]
    per_step = {PHASES[k]: sums[1 + k] / steps for k in range(6)}
    loop = sums[7] / steps
    rec = {"workload": wl.name, "build": "libmsa_trace.so (MSA_PHASE_TRACE)",
           "kernel_us_untraced_calls": plain_ms / n * 1e3, "kernel_us_traced_calls": traced_ms / n2 * 1e3,
           "wave_steps": int(steps), "clocks_per_step": loop, "phase_clocks_per_step": per_step,
           "mfma_clocks_per_step_per_simd": 2 * 32 * 32,
           "mfma_share_of_step": 2 * 32 * 32 / loop,
           "tflops_untraced": f / (plain_ms / n * 1e-3) / 1e12}
    print(json.dumps(rec))
    if args.report:
        lines = [f"# msa_prefill_kernel on {wl.name}: phase trace", "",
                 "Commands (from the repository root; the library is built on the build host, then run on an MI355X):",
                 "", "    python -m kv_cache_attention_msa_amd.csrc.build --phase-trace",
                 f"    python bench.py --phase-trace --steps {args.steps} --report {args.report}", "",
                 "The measurement build reads the shader clock (`s_memtime`, between scheduling fences) at every phase",
                 "boundary of every 64-key step and sums the differences per work item and wave; reading the clock",
                 "waits for it, so traced steps run longer than plain ones (kernel times below).", "",
                 f"- kernel time, same build: {rec['kernel_us_untraced_calls']:.1f} us with tracing off, "
                 f"{rec['kernel_us_traced_calls']:.1f} us with it on ({args.steps} calls each)",
                 f"- wave-steps traced: {int(steps)} ({args.steps} calls x {n_items} work items x their waves x their "
                 f"steps)",
                 f"- clocks per step and wave: {loop:.0f}; the two waves of a SIMD need 2 x 32 MFMAs x 32 clocks = "
                 f"2048 MFMA clocks per step, {100 * rec['mfma_share_of_step']:.0f} % of it", "",
                 "| phase | clocks per step | share |", "|---|---|---|"]
        for k, v in per_step.items():
            lines.append(f"| {k} | {v:.0f} | {100 * v / loop:.0f} % |")
        with open(args.report, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {args.report}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "write", "heavy", "mixed", "mixed_prefill", "mixed_decode",
                                       "tiny"], help="time one workload only (profiler runs)")
    ap.add_argument("--copy-bytes", type=int, help="run a plain copy kernel of this size (counter calibration)")
    ap.add_argument("--report", help="write a profile summary from rocprofv3 CSV output (no GPU needed)")
    ap.add_argument("--key", choices=["prefill", "decode", "write"])
    ap.add_argument("--kernel", default="msa_prefill_kernel")
    ap.add_argument("--units", default="")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-kernel", default="neg_kernel")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--notes", action="append", default=[])
    ap.add_argument("--latency-model", action="store_true", help="calibrate the Eq. 5 latency model on this GPU")
    ap.add_argument("--latency-out", help="with --latency-model: also write the full result (JSON) here")
    ap.add_argument("--latency-batch", type=int, default=16, help="requests per step for --latency-model")
    ap.add_argument("--latency-report", help="summarise a --latency-out JSON into --report (no GPU needed)")
    ap.add_argument("--phase-trace", action="store_true",
                    help="per-phase clocks of the chunk kernel (needs libmsa_trace.so: csrc.build --phase-trace)")
    ap.add_argument("--evict-sweep", action="store_true",
                    help="eviction time against 4-10 x 10^3 cached blocks (host only; with --report, a summary)")
    args = ap.parse_args()
    if args.phase_trace:
        phase_trace_run(args)
        return
    if args.latency_report:
        latency_report(args.latency_report, args.report,
                       args.command[0] if args.command else f"python bench.py --latency-model --latency-out {args.latency_report}")
        return
    if args.evict_sweep:
        evict_sweep(args.report)
        return
    if args.report:
        write_report(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: MSA runs on a single MI355X here (no multi-GPU path).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_kernel_run(args.copy_bytes)
        return
    if args.latency_model:
        latency_model_run(args)
        return
    if args.only == "write":
        import workloads as W
        wl = W.config5()
        fresh = W.fresh_kv(wl, seed=5)
        ms, k_warm, k_cold, k_n = run_write(wl, fresh, args.steps, args.warmup)
        print(json.dumps({"workload": wl.name + "_fresh", "ms_per_step": ms, "kernel_avg_ms": k_cold,
                          "kernel_warm_ms": k_warm, "launches": k_n}), flush=True)
        return
    if args.only:
        import kv_cache_attention_msa_amd as msa
        import workloads as W
        if args.only in ("mixed", "mixed_prefill", "mixed_decode"):
            wl = W.config5()
            pre, dec = W.mixed_parts(wl)
            if args.only != "mixed":
                wl = W.subset(wl, pre if args.only == "mixed_prefill" else dec, wl.name + "_" + args.only[6:] + "_part")
        else:
            wl = {"prefill": W.config2, "decode": W.config3, "heavy": W.config4, "tiny": W.config1}[args.only]()
        kind = {"decode": msa.KERNEL_DECODE, "mixed_decode": msa.KERNEL_DECODE,
                "tiny": msa.KERNEL_FP32}.get(args.only, msa.KERNEL_PREFILL)
        ms, times, plan_ms = run_workload(wl, args.steps, args.warmup, kind)
        k_ms, k_n = times[kind]
        print(json.dumps({"workload": wl.name, "ms_per_step": ms, "kernel_avg_ms": k_ms / max(k_n, 1),
                          "launches": k_n}), flush=True)
        return

    import torch
    import kv_cache_attention_msa_amd as msa
    import workloads as W

    msa.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = W.CONFIGS[args.config]()
    flops, nbytes = work_of(wl)
    counts, _ = visible_counts(wl)
    ms, times, plan_ms = run_workload(wl, args.steps, args.warmup, msa.KERNEL_PREFILL)
    roofline = mfma_roofline(wl, flops, times, args.steps)
    line = {
        "metric": METRIC, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "settle_s": SETTLE_S,
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": 16, "total_q": wl.total_q,
                   "segments": int(len(wl.segs)), "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                   "host_call_ms": plan_ms},
        "roofline": roofline,
    }
    if not args.no_secondary:
        line["secondary"] = decode_entry(W.config3(), args.steps, args.warmup)
        line["heavy"] = mfma_entry(W.config4(), args.steps, args.warmup)
        line["mixed"], line["kv_write"] = mixed_entries(W.config5(), args.steps, args.warmup)
        line["tiny"] = tiny_entry(W.config1(), args.steps, args.warmup)
    att = attainable_peaks()
    line["attainable"] = att
    for sr in rooflines(line):
        ref = {"mfma": "mfma_bf16_TFLOPs", "hbm": "hbm_gather_4KiB_GBps", "copy": "hbm_copy_GBps"}[sr.pop("_ref")]
        sr["frac_of_attainable"] = sr["achieved"] / att[ref] if sr.get("achieved") else None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, counts * wl.num_q_heads * 4 * wl.head_dim)
        if not args.no_secondary:
            line["cpu_baseline"]["other_workloads"] = cpu_oracle_configs()
    print(json.dumps(line), flush=True)


def rooflines(line):
    """Every roofline object of the report (headline and sub-entries)."""
    out = [line["roofline"]]
    for key in ("secondary", "heavy", "kv_write"):
        if key in line:
            out.append(line[key]["roofline"])
    if "mixed" in line:
        out += [line["mixed"]["prefill_part"]["roofline"], line["mixed"]["decode_part"]["roofline"]]
    return out


def mfma_roofline(wl, flops, times, steps):
    """Roofline of the chunk (MFMA) kernel: one launch processes the whole workload."""
    import kv_cache_attention_msa_amd as msa
    pre_ms, pre_n = times[msa.KERNEL_PREFILL]
    dec_n = times[msa.KERNEL_DECODE][1]
    mrg_ms, mrg_n = times[msa.KERNEL_MERGE]
    k_avg = pre_ms / max(pre_n, 1)
    achieved = flops / (k_avg * 1e-3) / 1e12 if pre_n else None
    return {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS if achieved else None, "gate": GATE_MFMA,
            "traffic": traffic_for("prefill", wl.name),
            "kernel": "msa_prefill (bf16 MFMA)", "kernel_ms": k_avg, "kernel_ms_dist": times["dist"],
            "merge_ms": mrg_ms / mrg_n if mrg_n else 0.0, "launches_per_step": (pre_n + dec_n + mrg_n) / steps,
            "_ref": "mfma"}


def hbm_roofline(wl, nbytes, times, kind_key="decode"):
    """Roofline of the decode (HBM) kernel."""
    import kv_cache_attention_msa_amd as msa
    d_ms, d_n = times[msa.KERNEL_DECODE]
    m_ms, m_n = times[msa.KERNEL_MERGE]
    d_avg = d_ms / max(d_n, 1)
    ach = nbytes / (d_avg * 1e-3) / 1e9 if d_n else None
    r = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": ach / PEAK_HBM_GBS if ach else None, "gate": GATE_HBM,
         "traffic": traffic_for(kind_key, wl.name), "kernel": "msa_decode",
         "kernel_ms": d_avg, "kernel_ms_dist": times["dist"], "merge_ms": m_ms / m_n if m_n else 0.0, "_ref": "hbm"}
    if "cold_dist" in times:
        r["kernel_ms_dist_cold"] = times["cold_dist"]
    return r


def decode_entry(wl, steps, warmup):
    import kv_cache_attention_msa_amd as msa
    f, b = work_of(wl)
    ms, t, plan = run_workload(wl, steps, warmup, msa.KERNEL_DECODE, cold=True)
    return {"workload": wl.name, "metric": "decode HBM GB/s", "value": b / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "ms_per_step": ms, "algorithmic_bytes": b, "algorithmic_flops": f, "host_call_ms": plan,
            "roofline": hbm_roofline(wl, b, t)}


def mfma_entry(wl, steps, warmup):
    import kv_cache_attention_msa_amd as msa
    f, b = work_of(wl)
    ms, t, plan = run_workload(wl, steps, warmup, msa.KERNEL_PREFILL)
    return {"workload": wl.name, "metric": "MSA TFLOP/s", "value": f / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "ms_per_step": ms, "algorithmic_flops": f, "algorithmic_bytes": b, "host_call_ms": plan,
            "roofline": mfma_roofline(wl, f, t, steps)}


def mixed_entries(wl, steps, warmup):
    """The mixed batch: the whole batch against T_roof = max(F / F_peak, B / B_peak),
    its prefill-only and decode-only parts each against their own roofline
    (same pool, same descriptors, timed as separate calls), and the KV write of
    its fresh rows."""
    import torch
    import kv_cache_attention_msa_amd as msa
    import workloads as W
    kv = wl.dense_pool("cuda")
    f, b = work_of(wl)
    ms, t, plan = run_workload(wl, steps, warmup, msa.KERNEL_PREFILL, pool_kv=kv)
    dev_ms = sum(t[k][0] for k in (msa.KERNEL_PREFILL, msa.KERNEL_DECODE, msa.KERNEL_MERGE, msa.KERNEL_UPLOAD)) / steps
    t_roof = max(f / (PEAK_BF16_TFLOPS * 1e12), b / (PEAK_HBM_GBS * 1e9)) * 1e3
    per_kernel = {name: (t[k][0] / t[k][1] if t[k][1] else 0.0)
                  for name, k in (("chunk_ms", msa.KERNEL_PREFILL), ("decode_ms", msa.KERNEL_DECODE),
                                  ("merge_ms", msa.KERNEL_MERGE), ("upload_ms", msa.KERNEL_UPLOAD))}
    pre_seqs, dec_seqs = W.mixed_parts(wl)
    wp = W.subset(wl, pre_seqs, wl.name + "_prefill_part")
    wd = W.subset(wl, dec_seqs, wl.name + "_decode_part")
    fp, bp = work_of(wp)
    msp, tp, _ = run_workload(wp, steps, warmup, msa.KERNEL_PREFILL, pool_kv=kv)
    fd, bd = work_of(wd)
    msd, td, _ = run_workload(wd, steps, warmup, msa.KERNEL_DECODE, pool_kv=kv)
    mixed = {"workload": wl.name, "metric": "T_roof / T", "ms_per_step": ms, "device_ms_per_step": dev_ms,
             "algorithmic_flops": f, "algorithmic_bytes": b, "T_roof_ms": t_roof,
             "value": t_roof / ms, "roof_frac_device": t_roof / dev_ms, "kernels": per_kernel, "host_call_ms": plan,
             "prefill_part": {"workload": wp.name, "sequences": len(pre_seqs), "total_q": wp.total_q,
                              "ms_per_step": msp, "algorithmic_flops": fp, "algorithmic_bytes": bp,
                              "roofline": mfma_roofline(wp, fp, tp, steps)},
             "decode_part": {"workload": wd.name, "sequences": len(dec_seqs), "ms_per_step": msd,
                             "algorithmic_flops": fd, "algorithmic_bytes": bd,
                             "roofline": hbm_roofline(wd, bd, td)}}
    fresh = W.fresh_kv(wl, seed=5)
    b5 = write_bytes(wl, fresh)
    ms5, k5w, k5, n5 = run_write(wl, fresh, steps, warmup, pool_kv=kv)
    ach5 = b5 / (k5 * 1e-3) / 1e9 if n5 else None
    write = {
        "workload": wl.name + "_fresh", "metric": "KV write HBM GB/s", "value": b5 / (ms5 * 1e-3) / 1e9,
        "unit": "GB/s", "ms_per_step": ms5, "algorithmic_bytes": b5, "segments": int(len(fresh.segs)),
        "rows": fresh.rows,
        "roofline": {"bound": "hbm", "achieved": ach5, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach5 / PEAK_HBM_GBS if ach5 else None,
                     "traffic": traffic_for("write", wl.name + "_fresh"), "kernel": "msa_write",
                     "kernel_ms": k5, "cache": "cold (1 GiB read between calls evicts the Infinity Cache)",
                     "kernel_warm_ms": k5w, "achieved_warm": b5 / (k5w * 1e-3) / 1e9 if n5 else None,
                     "kernel_ms_dist_cold": run_write.dists["cold"],
                     "kernel_ms_dist_warm": run_write.dists["warm"], "_ref": "copy"},
    }
    del kv
    torch.cuda.empty_cache()
    return mixed, write


def tiny_entry(wl, steps, warmup):
    """The tiny fp32 case: launch-latency bound, so time only (no roofline fraction)."""
    import kv_cache_attention_msa_amd as msa
    f, b = work_of(wl)
    ms, t, plan = run_workload(wl, steps, warmup, msa.KERNEL_FP32)
    k_ms, k_n = t[msa.KERNEL_FP32]
    return {"workload": wl.name, "dtype": "f32", "ms_per_step": ms, "kernel_ms": k_ms / max(k_n, 1),
            "kernel_ms_dist": t["dist"], "algorithmic_flops": f, "algorithmic_bytes": b, "host_call_ms": plan}


if __name__ == "__main__":
    main()
