// C ABI of libmsa: pool lifetime, per-call plan upload and kernel launches.
//
// One msa_forward call:
//   1. checks every argument and builds the plan on the host (no HIP call
//      before this succeeds, so an error leaves the stream untouched);
//   2. packs the plan (block list, query positions, work and merge items) into
//      the next pinned, device-mapped staging buffer of a small ring;
//   3. enqueues on the caller's stream: a copy kernel that moves the plan into
//      the pool's device plan buffer, the prefill, decode and fp32 kernels for
//      the items of each kind, then the merge kernel when some tile was split
//      over KV.  Everything is on the caller's stream, so consecutive calls
//      are ordered without cross-stream events.
//
// msa_write_kv uses the same staging and upload for its destination block
// list, then one copy kernel that places the fresh K/V rows.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <utility>

#include "msa_internal.h"

using namespace msa;

namespace {

thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_error(hipError_t e, const char* what) {
  return set_error(MSA_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

#define MSA_HIP(call)                                         \
  do {                                                        \
    hipError_t e_ = (call);                                   \
    if (e_ != hipSuccess) return hip_error(e_, #call);        \
  } while (0)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Restores the calling thread's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && (prev == dev || hipSetDevice(dev) == hipSuccess)) ok = true;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

struct TimingRecord {
  int kind;
  hipEvent_t start, stop;
};

}  // namespace

namespace msa {
// Error reporting for the library's other host sources.
int set_error_msg(int code, const std::string& msg) { return set_error(code, "%s", msg.c_str()); }
}  // namespace msa

struct msa_pool {
  msa_pool_desc desc{};
  void* k = nullptr;
  void* v = nullptr;
  bool owns_kv = false;
  int num_cus = 0;  // 0: not queried yet

  // options
  bool timing = false;
  bool check_ids = false;
  void* trace = nullptr;     // MSA_OPT_PHASE_TRACE buffer (tracing builds)
  int32_t split_blocks = 0;
  int32_t num_cus_override = 0;
  int32_t chunk_waves = 0;   // MSA_OPT_CHUNK_WAVES

  // Plan upload: call n packs its plan into pinned, device-mapped staging
  // buffer n % kSlots; a small kernel on the caller's stream copies it into the
  // device plan buffer ahead of the attention kernels (same queue, so no
  // cross-engine hand-off).  A staging buffer is rewritten only once the copy
  // that read it has run (event), which in steady state is long done.
  static constexpr int kSlots = 3;
  void* h_stage[kSlots] = {};
  void* h_stage_dev[kSlots] = {};      // device address of the same pinned memory
  size_t stage_bytes[kSlots] = {};
  hipEvent_t stage_done[kSlots] = {};
  bool stage_pending[kSlots] = {};
  int next_slot = 0;
  int last_slot = 0;                   // slot of the most recent upload
  void* d_plan = nullptr;
  size_t plan_cap = 0;
  // partial results of KV-split tiles
  void* d_part = nullptr;
  size_t part_bytes = 0;
  hipStream_t last_stream = nullptr;
  bool used = false;

  // timing
  std::vector<TimingRecord> records;
  std::vector<hipEvent_t> spare_events;
  double total_ms[kNumKinds] = {};
  int64_t launches[kNumKinds] = {};
  static constexpr size_t kMaxSamples = 1 << 16;  // per kind; the oldest are dropped beyond this
  std::vector<float> samples[kNumKinds];

  Plan plan;
  std::vector<BlockEntry> write_entries;  // msa_write_kv's block list
};

namespace {

int take_event(msa_pool* p, hipEvent_t* ev) {
  if (!p->spare_events.empty()) {
    *ev = p->spare_events.back();
    p->spare_events.pop_back();
    return MSA_OK;
  }
  MSA_HIP(hipEventCreate(ev));
  return MSA_OK;
}

int collect_timing(msa_pool* p) {
  for (auto& r : p->records) {
    MSA_HIP(hipEventSynchronize(r.stop));
    float ms = 0.f;
    MSA_HIP(hipEventElapsedTime(&ms, r.start, r.stop));
    p->total_ms[r.kind] += ms;
    p->launches[r.kind] += 1;
    std::vector<float>& v = p->samples[r.kind];
    if (v.size() >= msa_pool::kMaxSamples) v.erase(v.begin(), v.begin() + v.size() / 2);
    v.push_back(ms);
    p->spare_events.push_back(r.start);
    p->spare_events.push_back(r.stop);
  }
  p->records.clear();
  return MSA_OK;
}

// Launch one kernel kind, bracketed by events when timing is on.
template <typename F>
int timed_launch(msa_pool* p, int kind, hipStream_t stream, F&& launch) {
  TimingRecord rec{kind, nullptr, nullptr};
  if (p->timing) {
    int rc = take_event(p, &rec.start);
    if (rc) return rc;
    rc = take_event(p, &rec.stop);
    if (rc) return rc;
    MSA_HIP(hipEventRecord(rec.start, stream));
  }
  int e = launch();
  if (e != hipSuccess) return hip_error((hipError_t)e, "kernel launch");
  if (p->timing) {
    MSA_HIP(hipEventRecord(rec.stop, stream));
    p->records.push_back(rec);
    if (p->records.size() > 4096) return collect_timing(p);
  }
  return MSA_OK;
}

int grow_device(void** ptr, size_t* cap, size_t bytes, const char* what) {
  if (bytes <= *cap) return MSA_OK;
  const size_t want = align_up(std::max(bytes, *cap + *cap / 2), size_t(1) << 16);
  if (*ptr) {
    MSA_HIP(hipFree(*ptr));
    *ptr = nullptr;
    *cap = 0;
  }
  hipError_t e = hipMalloc(ptr, want);
  if (e != hipSuccess) {
    *ptr = nullptr;
    (void)hipGetLastError();
    return set_error(MSA_ERR_OOM, "%s hipMalloc(%zu) failed: %s", what, want, hipGetErrorString(e));
  }
  *cap = want;
  return MSA_OK;
}

// Device buffers read by kernels of earlier calls are only replaced once the
// streams that used them have drained.
int ensure_device(msa_pool* p, void** ptr, size_t* cap, size_t bytes, hipStream_t stream, const char* what) {
  if (bytes <= *cap) return MSA_OK;
  if (*ptr) {
    if (p->used) MSA_HIP(hipStreamSynchronize(p->last_stream));
    MSA_HIP(hipStreamSynchronize(stream));
  }
  return grow_device(ptr, cap, bytes, what);
}

int ensure_stage(msa_pool* p, int slot, size_t bytes) {
  if (!p->stage_done[slot]) MSA_HIP(hipEventCreateWithFlags(&p->stage_done[slot], hipEventDisableTiming));
  if (p->stage_pending[slot]) {
    MSA_HIP(hipEventSynchronize(p->stage_done[slot]));
    p->stage_pending[slot] = false;
  }
  if (bytes <= p->stage_bytes[slot]) return MSA_OK;
  size_t want = align_up(std::max(bytes, p->stage_bytes[slot] * 3 / 2), size_t(1) << 16);
  if (p->h_stage[slot]) {
    MSA_HIP(hipHostFree(p->h_stage[slot]));
    p->h_stage[slot] = p->h_stage_dev[slot] = nullptr;
    p->stage_bytes[slot] = 0;
  }
  hipError_t e = hipHostMalloc(&p->h_stage[slot], want, hipHostMallocMapped);
  if (e != hipSuccess) {
    p->h_stage[slot] = nullptr;
    (void)hipGetLastError();
    return set_error(MSA_ERR_OOM, "pinned hipHostMalloc(%zu) failed: %s", want, hipGetErrorString(e));
  }
  MSA_HIP(hipHostGetDevicePointer(&p->h_stage_dev[slot], p->h_stage[slot], 0));
  p->stage_bytes[slot] = want;
  return MSA_OK;
}

size_t elem_size(int dtype) { return dtype == MSA_FP32 ? 4 : 2; }

// Packs `bytes` of per-call data (written by `fill` into host memory) into
// the next staging slot and enqueues its copy into the device plan buffer on
// `stream`; the first n_blocks BlockEntry of the data get their block-table
// index resolved to a pool block id on the way.
template <typename Fill>
int stage_and_upload(msa_pool* p, hipStream_t stream, size_t bytes, int32_t n_blocks,
                     const int32_t* block_table, Fill&& fill) {
  int rc = ensure_device(p, &p->d_plan, &p->plan_cap, bytes, stream, "plan buffer");
  if (rc) return rc;
  const int slot = p->next_slot;
  p->next_slot = (p->next_slot + 1) % msa_pool::kSlots;
  p->last_slot = slot;
  rc = ensure_stage(p, slot, bytes);
  if (rc) return rc;
  fill((char*)p->h_stage[slot]);
  rc = timed_launch(p, kUpload, stream, [&]() {
    return launch_upload(p->h_stage_dev[slot], p->d_plan, bytes, n_blocks, block_table, p->desc.num_blocks,
                         stream);
  });
  if (rc) return rc;
  MSA_HIP(hipEventRecord(p->stage_done[slot], stream));
  p->stage_pending[slot] = true;
  p->used = true;
  p->last_stream = stream;
  return MSA_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// ---- one attention call: checks, plan layout, packing and launches ----------

// Argument checks and planning, shared by both attention entry points.  No
// HIP call is made; *empty is set when there is nothing to enqueue.
int prepare_call(msa_pool* p, const msa_seg_desc* desc, const void* q, const int32_t* block_table, const void* out,
                 const float* lse, bool* empty) {
  if (!p) return set_error(MSA_ERR_INVALID_ARG, "pool is NULL");
  if (!desc) return set_error(MSA_ERR_INVALID_ARG, "seg_desc is NULL");
  PlanConfig cfg;
  cfg.num_kv_heads = p->desc.num_kv_heads;
  cfg.head_dim = p->desc.head_dim;
  cfg.dtype = p->desc.dtype;
  cfg.num_cus = p->num_cus_override > 0 ? p->num_cus_override : (p->num_cus > 0 ? p->num_cus : 256);
  cfg.split_blocks = p->split_blocks;
  cfg.chunk_waves = p->chunk_waves;
  std::string err;
  int rc = build_plan(desc, cfg, p->plan, err);
  if (rc) return set_error(rc, "%s", err.c_str());
  const Plan& plan = p->plan;
  if (plan.total_q > 0 && (!q || !out)) return set_error(MSA_ERR_INVALID_ARG, "q or out is NULL");
  if (!plan.blocks.empty() && !block_table) return set_error(MSA_ERR_INVALID_ARG, "block_table is NULL");
  if (plan.total_q > 0 && (q == out || (const void*)lse == q || (const void*)lse == out))
    return set_error(MSA_ERR_INVALID_ARG, "q, out and lse must not alias");
  *empty = plan.total_q == 0;
  return MSA_OK;
}

// On the first call, learn the device's compute-unit count and plan again if
// it differs from the count assumed.  The device must be current.
int refresh_cus(msa_pool* p, const msa_seg_desc* desc) {
  if (p->num_cus != 0) return MSA_OK;
  int n = 0;
  MSA_HIP(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, p->desc.device));
  const int assumed = p->num_cus_override > 0 ? p->num_cus_override : 256;
  p->num_cus = n > 0 ? n : 256;
  if (p->num_cus_override == 0 && p->num_cus != assumed) {
    PlanConfig cfg;
    cfg.num_kv_heads = p->desc.num_kv_heads;
    cfg.head_dim = p->desc.head_dim;
    cfg.dtype = p->desc.dtype;
    cfg.num_cus = p->num_cus;
    cfg.split_blocks = p->split_blocks;
    cfg.chunk_waves = p->chunk_waves;
    std::string err;
    int rc = build_plan(desc, cfg, p->plan, err);
    if (rc) return set_error(rc, "%s", err.c_str());
  }
  return MSA_OK;
}

// Where each part of a call's plan sits in the packed plan buffer, and the
// size of its partial-result area.
struct PlanLayout {
  size_t off_blocks, off_qpos, off_items[3], off_merge, off_check, plan_bytes;
  size_t off_part_lse, part_bytes;
};

// The block list is followed by kBlockPad zero entries so that a kernel may
// always read the entries of a step (their valid counts are ignored).
constexpr size_t kBlockPad = 4;

// Two result words of the optional block-id check (count, smallest bad
// block-table index) close every packed plan; the host writes their start
// values and the upload copies them into device memory.
constexpr size_t kCheckBytes = 256;

void pack_check_words(char* h) {
  const int32_t init[2] = {0, INT32_MAX};
  memset(h, 0, kCheckBytes);
  memcpy(h, init, sizeof(init));
}

// With MSA_OPT_CHECK_BLOCK_IDS: after the upload, count the block-list entries
// whose block-table entry is out of range (reading the host-packed list at
// `src`), read the result back and fail the call if there is any.  The call
// then has enqueued only the upload (into the library's own buffer).
int check_block_ids(msa_pool* p, hipStream_t stream, const void* src, int32_t n_blocks, const int32_t* block_table,
                    int32_t* d_result) {
  int e = launch_check_ids(src, n_blocks, block_table, p->desc.num_blocks, d_result, stream);
  if (e != hipSuccess) return hip_error((hipError_t)e, "kernel launch");
  int32_t r[2] = {0, 0};
  MSA_HIP(hipMemcpyAsync(r, d_result, sizeof(r), hipMemcpyDeviceToHost, stream));
  MSA_HIP(hipStreamSynchronize(stream));
  if (r[0] != 0)
    return set_error(MSA_ERR_INVALID_ARG, "%d block-list entries name pool block ids outside [0, %d); the first is "
                     "block_table[%d]", r[0], p->desc.num_blocks, r[1]);
  return MSA_OK;
}

PlanLayout plan_layout(const Plan& plan, int D) {
  PlanLayout L{};
  size_t off = 0;
  L.off_blocks = off;
  off = align_up(off + (plan.blocks.size() + kBlockPad) * sizeof(BlockEntry), 256);
  L.off_qpos = off;
  off = align_up(off + plan.q_pos.size() * sizeof(int32_t), 256);
  for (int k = 0; k < 3; ++k) {
    L.off_items[k] = off;
    off = align_up(off + plan.items[k].size() * sizeof(WorkItem), 256);
  }
  L.off_merge = off;
  off = align_up(off + plan.merges.size() * sizeof(MergeItem), 256);
  L.off_check = off;
  off += kCheckBytes;
  L.plan_bytes = off;
  L.off_part_lse = align_up((size_t)plan.part_rows * D * sizeof(float), 256);
  L.part_bytes = plan.part_rows > 0 ? L.off_part_lse + align_up((size_t)plan.part_rows * sizeof(float), 256) : 0;
  return L;
}

void pack_plan(const Plan& plan, const PlanLayout& L, char* h) {
  if (!plan.blocks.empty()) memcpy(h + L.off_blocks, plan.blocks.data(), plan.blocks.size() * sizeof(BlockEntry));
  memset(h + L.off_blocks + plan.blocks.size() * sizeof(BlockEntry), 0, kBlockPad * sizeof(BlockEntry));
  memcpy(h + L.off_qpos, plan.q_pos.data(), plan.q_pos.size() * sizeof(int32_t));
  for (int k = 0; k < 3; ++k)
    if (!plan.items[k].empty())
      memcpy(h + L.off_items[k], plan.items[k].data(), plan.items[k].size() * sizeof(WorkItem));
  if (!plan.merges.empty()) memcpy(h + L.off_merge, plan.merges.data(), plan.merges.size() * sizeof(MergeItem));
  pack_check_words(h + L.off_check);
}

// Enqueue the attention kernels of a planned call whose plan is in device
// memory at `dplan` (block ids resolved) and whose partials go to `dpart`.
int launch_attention(msa_pool* p, const msa_seg_desc* desc, const PlanLayout& L, char* dplan, char* dpart,
                     const void* q, void* out, float* lse, hipStream_t stream, bool timed) {
  const Plan& plan = p->plan;
  const int D = p->desc.head_dim;
  KernelArgs a{};
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.k = p->k;
  a.v = p->v;
  a.blocks = (const BlockEntry*)(dplan + L.off_blocks);
  a.q_pos = (const int32_t*)(dplan + L.off_qpos);
  a.merges = (const MergeItem*)(dplan + L.off_merge);
  a.n_merges = (int32_t)plan.merges.size();
  a.part_o = (float*)dpart;
  a.part_lse = dpart ? (float*)(dpart + L.off_part_lse) : nullptr;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = p->desc.num_kv_heads;
  a.group = desc->num_q_heads / p->desc.num_kv_heads;
  a.causal = desc->causal;
  const float scale = desc->scale != 0.f ? desc->scale : 1.0f / std::sqrt((float)D);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.trace = (unsigned long long*)p->trace;
  auto launch = [&](int kind, auto&& fn) -> int {
    if (timed) return timed_launch(p, kind, stream, fn);
    const int e = fn();
    return e != hipSuccess ? hip_error((hipError_t)e, "kernel launch") : MSA_OK;
  };
  for (int k = 0; k < 3; ++k) {
    if (plan.items[k].empty()) continue;
    a.items = (const WorkItem*)(dplan + L.off_items[k]);
    a.n_items = (int32_t)plan.items[k].size();
    a.max_mrows = plan.max_mrows[k];
    a.stream_kv = plan.stream_kv[k];
    const int rc = launch(k, [&]() {
      if (k == kPrefill) return launch_prefill(a, D, plan.chunk_waves, stream);
      if (k == kDecode) return launch_decode(a, D, stream);
      return launch_fp32(a, D, stream);
    });
    if (rc) return rc;
  }
  if (!plan.merges.empty()) {
    a.items = nullptr;
    a.n_items = 0;
    a.max_mrows = 0;
    for (const MergeItem& m : plan.merges) a.max_mrows = std::max(a.max_mrows, m.n_mrows);
    const int rc = launch(kMerge, [&]() { return launch_merge(a, D, p->desc.dtype, stream); });
    if (rc) return rc;
  }
  return MSA_OK;
}

}  // namespace

extern "C" {

const char* msa_last_error(void) { return g_last_error.c_str(); }

int msa_create_pool(const msa_pool_desc* desc, void* k_base, void* v_base, msa_pool** out) {
  if (!desc || !out) return set_error(MSA_ERR_INVALID_ARG, "desc or out is NULL");
  *out = nullptr;
  if (desc->num_blocks <= 0 || desc->num_kv_heads <= 0)
    return set_error(MSA_ERR_INVALID_ARG, "num_blocks and num_kv_heads must be > 0");
  if (desc->num_blocks > kMaxPoolBlocks)
    return set_error(MSA_ERR_UNSUPPORTED, "num_blocks %d exceeds %d", desc->num_blocks, kMaxPoolBlocks);
  if (desc->block_size != MSA_BLOCK_SIZE)
    return set_error(MSA_ERR_UNSUPPORTED, "block_size %d is not supported (16)", desc->block_size);
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return set_error(MSA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", desc->head_dim);
  if (desc->dtype != MSA_BF16 && desc->dtype != MSA_FP32)
    return set_error(MSA_ERR_UNSUPPORTED, "dtype %d is not supported", desc->dtype);
  if (desc->device < 0) return set_error(MSA_ERR_INVALID_ARG, "device %d < 0", desc->device);
  if ((k_base == nullptr) != (v_base == nullptr))
    return set_error(MSA_ERR_INVALID_ARG, "give both k_base and v_base, or neither");
  msa_pool* p = new (std::nothrow) msa_pool();
  if (!p) return set_error(MSA_ERR_OOM, "host allocation failed");
  p->desc = *desc;
  if (k_base) {
    p->k = k_base;
    p->v = v_base;
  } else {
    DeviceGuard g(desc->device);
    if (!g.ok) {
      delete p;
      return set_error(MSA_ERR_HIP, "cannot select device %d", desc->device);
    }
    const size_t bytes = (size_t)desc->num_blocks * desc->num_kv_heads * MSA_BLOCK_SIZE *
                         desc->head_dim * elem_size(desc->dtype);
    if (hipMalloc(&p->k, bytes) != hipSuccess || hipMalloc(&p->v, bytes) != hipSuccess) {
      (void)hipGetLastError();
      if (p->k) (void)hipFree(p->k);
      delete p;
      return set_error(MSA_ERR_OOM, "pool hipMalloc of 2 x %zu bytes failed", bytes);
    }
    p->owns_kv = true;
  }
  *out = p;
  return MSA_OK;
}

int msa_pool_kv_ptrs(const msa_pool* pool, void** k, void** v) {
  if (!pool || !k || !v) return set_error(MSA_ERR_INVALID_ARG, "NULL argument");
  *k = pool->k;
  *v = pool->v;
  return MSA_OK;
}

int msa_destroy_pool(msa_pool* p) {
  if (!p) return MSA_OK;
  int rc = MSA_OK;
  const bool touched = p->used || p->owns_kv || p->d_plan || p->d_part || p->h_stage[0];
  if (touched) {
    DeviceGuard g(p->desc.device);
    if (p->used && hipStreamSynchronize(p->last_stream) != hipSuccess) rc = MSA_ERR_HIP;
    for (auto& r : p->records) {
      (void)hipEventDestroy(r.start);
      (void)hipEventDestroy(r.stop);
    }
    for (auto e : p->spare_events) (void)hipEventDestroy(e);
    for (int s = 0; s < msa_pool::kSlots; ++s) {
      if (p->stage_done[s]) (void)hipEventDestroy(p->stage_done[s]);
      if (p->h_stage[s]) (void)hipHostFree(p->h_stage[s]);
    }
    if (p->d_plan) (void)hipFree(p->d_plan);
    if (p->d_part) (void)hipFree(p->d_part);
    if (p->owns_kv) {
      (void)hipFree(p->k);
      (void)hipFree(p->v);
    }
  }
  delete p;
  if (rc) return set_error(rc, "stream synchronisation failed while destroying the pool");
  return MSA_OK;
}

int msa_pool_set_option(msa_pool* p, int32_t option, int64_t value) {
  if (!p) return set_error(MSA_ERR_INVALID_ARG, "pool is NULL");
  switch (option) {
    case MSA_OPT_TIMING: p->timing = value != 0; return MSA_OK;
    case MSA_OPT_CHECK_BLOCK_IDS: p->check_ids = value != 0; return MSA_OK;
    case MSA_OPT_PHASE_TRACE:
#ifdef MSA_PHASE_TRACE
      p->trace = (void*)(uintptr_t)value;
      return MSA_OK;
#else
      if (value == 0) return MSA_OK;
      return set_error(MSA_ERR_UNSUPPORTED, "phase tracing needs the tracing build (libmsa_trace.so)");
#endif
    case MSA_OPT_SPLIT_BLOCKS:
      if (value < 0 || value > (1 << 30)) return set_error(MSA_ERR_INVALID_ARG, "bad split_blocks");
      p->split_blocks = (int32_t)value;
      return MSA_OK;
    case MSA_OPT_CHUNK_WAVES:
      if (value != 0 && value != 4 && value != 8) return set_error(MSA_ERR_INVALID_ARG, "chunk waves must be 0, 4 or 8");
      p->chunk_waves = (int32_t)value;
      return MSA_OK;
    case MSA_OPT_NUM_CUS:
      if (value < 0 || value > 65536) return set_error(MSA_ERR_INVALID_ARG, "bad num_cus");
      p->num_cus_override = (int32_t)value;
      return MSA_OK;
    default: return set_error(MSA_ERR_INVALID_ARG, "unknown option %d", option);
  }
}

int msa_pool_kernel_time(msa_pool* p, int32_t kind, double* total_ms, int64_t* launches, int32_t reset) {
  if (!p || !total_ms || !launches) return set_error(MSA_ERR_INVALID_ARG, "NULL argument");
  if (kind < 0 || kind >= kNumKinds) return set_error(MSA_ERR_INVALID_ARG, "bad kernel kind %d", kind);
  if (!p->records.empty()) {
    DeviceGuard g(p->desc.device);
    int rc = collect_timing(p);
    if (rc) return rc;
  }
  *total_ms = p->total_ms[kind];
  *launches = p->launches[kind];
  if (reset) {
    for (int k = 0; k < kNumKinds; ++k) {
      p->total_ms[k] = 0;
      p->launches[k] = 0;
      p->samples[k].clear();
    }
  }
  return MSA_OK;
}

int msa_pool_kernel_samples(msa_pool* p, int32_t kind, double* out, int32_t max, int32_t* n) {
  if (!p || !n || (max > 0 && !out)) return set_error(MSA_ERR_INVALID_ARG, "NULL argument");
  if (kind < 0 || kind >= kNumKinds) return set_error(MSA_ERR_INVALID_ARG, "bad kernel kind %d", kind);
  if (max < 0) return set_error(MSA_ERR_INVALID_ARG, "max < 0");
  if (!p->records.empty()) {
    DeviceGuard g(p->desc.device);
    int rc = collect_timing(p);
    if (rc) return rc;
  }
  const std::vector<float>& v = p->samples[kind];
  const size_t k = std::min(v.size(), (size_t)max);
  for (size_t i = 0; i < k; ++i) out[i] = v[v.size() - k + i];
  *n = (int32_t)k;
  return MSA_OK;
}

int msa_plan_debug(const msa_seg_desc* desc, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   int32_t num_cus, int32_t split_blocks, msa_plan_item* items, int32_t max_items,
                   int32_t* n_items, msa_plan_block* blocks, int32_t max_blocks, int32_t* n_blocks) {
  if (!n_items || !n_blocks) return set_error(MSA_ERR_INVALID_ARG, "n_items or n_blocks is NULL");
  if ((max_items > 0 && !items) || (max_blocks > 0 && !blocks))
    return set_error(MSA_ERR_INVALID_ARG, "NULL output array");
  PlanConfig cfg;
  cfg.num_kv_heads = num_kv_heads;
  cfg.head_dim = head_dim;
  cfg.dtype = dtype;
  cfg.num_cus = num_cus > 0 ? num_cus : 256;
  cfg.split_blocks = split_blocks;
  Plan plan;
  std::string err;
  int rc = build_plan(desc, cfg, plan, err);
  if (rc) return set_error(rc, "%s", err.c_str());
  int32_t n = 0;
  for (int k = 0; k < 3; ++k)
    for (const WorkItem& w : plan.items[k]) {
      if (n < max_items)
        items[n] = msa_plan_item{w.kind, w.seq, w.kv_head, w.q_row0, w.n_q, w.blk_begin, w.blk_end, w.part_row, k};
      ++n;
    }
  *n_items = n;
  const int32_t nb = (int32_t)plan.blocks.size();
  for (int32_t i = 0; i < std::min(nb, max_blocks); ++i) {
    const uint32_t bv = (uint32_t)plan.blocks[i].bt_valid;
    blocks[i] = msa_plan_block{(int32_t)(bv & ((1u << kBtIndexBits) - 1)), plan.blocks[i].pos0,
                               (int32_t)(bv >> kBtIndexBits) + 1};
  }
  *n_blocks = nb;
  return MSA_OK;
}

int msa_forward(const void* q, const msa_seg_desc* desc, const int32_t* block_table, msa_pool* p,
                void* out, float* lse, void* stream_) {
  bool empty = false;
  int rc = prepare_call(p, desc, q, block_table, out, lse, &empty);
  if (rc || empty) return rc;
  hipStream_t stream = (hipStream_t)stream_;
  DeviceGuard guard(p->desc.device);
  if (!guard.ok) return set_error(MSA_ERR_HIP, "cannot select device %d", p->desc.device);
  rc = refresh_cus(p, desc);
  if (rc) return rc;

  const Plan& plan = p->plan;
  const PlanLayout L = plan_layout(plan, p->desc.head_dim);
  if (L.part_bytes > 0) {
    rc = ensure_device(p, &p->d_part, &p->part_bytes, L.part_bytes, stream, "partial-result buffer");
    if (rc) return rc;
  }
  rc = stage_and_upload(p, stream, L.plan_bytes, (int32_t)plan.blocks.size(), block_table,
                        [&](char* h) { pack_plan(plan, L, h); });
  if (rc) return rc;
  if (p->check_ids) {
    rc = check_block_ids(p, stream, p->h_stage_dev[p->last_slot], (int32_t)plan.blocks.size(), block_table,
                         (int32_t*)((char*)p->d_plan + L.off_check));
    if (rc) return rc;
  }
  return launch_attention(p, desc, L, (char*)p->d_plan, (char*)p->d_part, q, out, lse, stream, p->timing);
}

int msa_forward_noalloc(const void* q, const msa_seg_desc* desc, const int32_t* block_table, msa_pool* p,
                        void* out, float* lse, void* stream_) {
  bool empty = false;
  int rc = prepare_call(p, desc, q, block_table, out, lse, &empty);
  if (rc || empty) return rc;
  {
    const PlanLayout L = plan_layout(p->plan, p->desc.head_dim);
    if (L.plan_bytes > kScratchPlanBytes || L.part_bytes > kScratchPartBytes)
      return set_error(MSA_ERR_WORKSPACE,
                       "call needs %zu plan bytes and %zu partial-result bytes; the fixed scratch holds at most "
                       "%zu and %zu",
                       L.plan_bytes, L.part_bytes, kScratchPlanBytes, kScratchPartBytes);
  }
  hipStream_t stream = (hipStream_t)stream_;
  DeviceGuard guard(p->desc.device);
  if (!guard.ok) return set_error(MSA_ERR_HIP, "cannot select device %d", p->desc.device);
  rc = refresh_cus(p, desc);
  if (rc) return rc;
  const Plan& plan = p->plan;
  const PlanLayout L = plan_layout(plan, p->desc.head_dim);
  if (L.plan_bytes > kScratchPlanBytes || L.part_bytes > kScratchPartBytes)
    return set_error(MSA_ERR_WORKSPACE, "plan for %d compute units exceeds the fixed scratch", p->num_cus);
  void* base = nullptr;
  std::string err;
  rc = scratch_address(p->desc.device, &base, err);
  if (rc) return set_error(rc, "%s", err.c_str());
  char* stage = (char*)base;                       // host copy of the packed plan
  char* dplan = stage + kScratchPlanBytes;          // the plan the kernels read
  char* dpart = dplan + kScratchPlanBytes;          // split partials

  // Pack into host memory of this thread and copy it into the scratch on the
  // stream.  A copy from pageable memory returns once its source has been
  // taken, so the host buffer is free again when the call returns.
  thread_local std::vector<char> host;
  if (host.size() < L.plan_bytes) host.resize(L.plan_bytes);
  pack_plan(plan, L, host.data());
  MSA_HIP(hipMemcpyAsync(stage, host.data(), L.plan_bytes, hipMemcpyHostToDevice, stream));
  int e = launch_upload(stage, dplan, L.plan_bytes, (int32_t)plan.blocks.size(), block_table, p->desc.num_blocks,
                        stream);
  if (e != hipSuccess) return hip_error((hipError_t)e, "kernel launch");
  if (p->check_ids) {
    rc = check_block_ids(p, stream, stage, (int32_t)plan.blocks.size(), block_table, (int32_t*)(dplan + L.off_check));
    if (rc) return rc;
  }
  return launch_attention(p, desc, L, dplan, dpart, q, out, lse, stream, false);
}

int msa_write_kv(msa_pool* p, const void* k_src, const void* v_src, int32_t num_src_rows, const msa_segment* segs,
                 const int32_t* src_rows, int32_t num_segs, const int32_t* block_table, int32_t block_table_len,
                 void* stream_) {
  // ---- host-side checks (no HIP call before they pass) ----
  if (!p) return set_error(MSA_ERR_INVALID_ARG, "pool is NULL");
  if (num_segs < 0 || num_src_rows < 0 || block_table_len < 0)
    return set_error(MSA_ERR_INVALID_ARG, "num_segs, num_src_rows and block_table_len must be >= 0");
  if (num_segs > 0 && (!segs || !src_rows)) return set_error(MSA_ERR_INVALID_ARG, "segs or src_rows is NULL");
  std::vector<std::pair<int32_t, int32_t>> bt_ranges;  // [bt_start, bt_end) of non-empty segments
  bt_ranges.reserve(num_segs);
  int64_t n_entries = 0;
  for (int32_t s = 0; s < num_segs; ++s) {
    const msa_segment& g = segs[s];
    if (g.len < 0 || g.bt_start < 0 || src_rows[s] < 0)
      return set_error(MSA_ERR_INVALID_ARG, "segment %d: len, bt_start and src_rows must be >= 0", s);
    if (g.len == 0) continue;
    const int64_t nb = (g.len + kBlock - 1) / kBlock;
    if ((int64_t)g.bt_start + nb > block_table_len)
      return set_error(MSA_ERR_INVALID_ARG, "segment %d: block-table range [%d, %lld) exceeds block_table_len %d", s,
                       g.bt_start, (long long)(g.bt_start + nb), block_table_len);
    if ((int64_t)src_rows[s] + g.len > num_src_rows)
      return set_error(MSA_ERR_INVALID_ARG, "segment %d: source rows [%d, %lld) exceed num_src_rows %d", s,
                       src_rows[s], (long long)src_rows[s] + g.len, num_src_rows);
    bt_ranges.emplace_back(g.bt_start, (int32_t)(g.bt_start + nb));
    n_entries += nb;
  }
  std::sort(bt_ranges.begin(), bt_ranges.end());
  for (size_t i = 1; i < bt_ranges.size(); ++i)
    if (bt_ranges[i].first < bt_ranges[i - 1].second)
      return set_error(MSA_ERR_INVALID_ARG, "two segments share block-table entry %d", bt_ranges[i].first);
  if (n_entries == 0) return MSA_OK;
  if (block_table_len > kMaxPoolBlocks)
    return set_error(MSA_ERR_WORKSPACE, "block_table_len %d exceeds %d", block_table_len, kMaxPoolBlocks);
  if (n_entries * p->desc.num_kv_heads > INT32_MAX)
    return set_error(MSA_ERR_WORKSPACE, "%lld (block, head) tiles exceed 2^31", (long long)(n_entries * p->desc.num_kv_heads));
  if (!k_src || !v_src || !block_table) return set_error(MSA_ERR_INVALID_ARG, "k_src, v_src or block_table is NULL");
  const size_t row_bytes = (size_t)p->desc.head_dim * elem_size(p->desc.dtype);
  const size_t src_bytes = (size_t)num_src_rows * p->desc.num_kv_heads * row_bytes;
  const size_t pool_bytes = (size_t)p->desc.num_blocks * p->desc.num_kv_heads * kBlock * row_bytes;
  if (ranges_overlap(k_src, src_bytes, v_src, src_bytes) || ranges_overlap(k_src, src_bytes, p->k, pool_bytes) ||
      ranges_overlap(k_src, src_bytes, p->v, pool_bytes) || ranges_overlap(v_src, src_bytes, p->k, pool_bytes) ||
      ranges_overlap(v_src, src_bytes, p->v, pool_bytes))
    return set_error(MSA_ERR_INVALID_ARG, "k_src and v_src must not overlap each other or the pool");

  // ---- block list: one entry per destination block, pos0 = source row of slot 0 ----
  std::vector<BlockEntry>& ent = p->write_entries;
  ent.clear();
  ent.reserve((size_t)n_entries);
  for (int32_t s = 0; s < num_segs; ++s) {
    const msa_segment& g = segs[s];
    for (int32_t j = 0; j * kBlock < g.len; ++j) {
      const int32_t valid = std::min(kBlock, g.len - j * kBlock);
      ent.push_back(BlockEntry{(int32_t)((uint32_t)(g.bt_start + j) | ((uint32_t)(valid - 1) << kBtIndexBits)),
                               src_rows[s] + j * kBlock});
    }
  }

  hipStream_t stream = (hipStream_t)stream_;
  DeviceGuard guard(p->desc.device);
  if (!guard.ok) return set_error(MSA_ERR_HIP, "cannot select device %d", p->desc.device);
  const size_t off_check = align_up(ent.size() * sizeof(BlockEntry), 256);
  const size_t bytes = off_check + kCheckBytes;
  int rc = stage_and_upload(p, stream, bytes, (int32_t)ent.size(), block_table, [&](char* h) {
    memcpy(h, ent.data(), ent.size() * sizeof(BlockEntry));
    memset(h + ent.size() * sizeof(BlockEntry), 0, off_check - ent.size() * sizeof(BlockEntry));
    pack_check_words(h + off_check);
  });
  if (rc) return rc;
  if (p->check_ids) {
    rc = check_block_ids(p, stream, p->h_stage_dev[p->last_slot], (int32_t)ent.size(), block_table,
                         (int32_t*)((char*)p->d_plan + off_check));
    if (rc) return rc;
  }
  WriteArgs a{};
  a.k_src = k_src;
  a.v_src = v_src;
  a.k = p->k;
  a.v = p->v;
  a.blocks = (const BlockEntry*)p->d_plan;
  a.n_entries = (int32_t)ent.size();
  a.num_kv_heads = p->desc.num_kv_heads;
  return timed_launch(p, kWrite, stream, [&]() { return launch_write(a, (int)row_bytes, stream); });
}

}  // extern "C"
