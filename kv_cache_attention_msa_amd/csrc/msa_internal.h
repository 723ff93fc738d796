// Internal types shared by the host runtime (planner, pool) and the HIP kernels.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "msa.h"

namespace msa {

constexpr int kBlock = MSA_BLOCK_SIZE;
constexpr int kPrefillMRows = 128;   // (query row, head-in-group) pairs per prefill tile (4 waves)
constexpr int kPrefillMRowsWide = 256;  // the same with 8-wave work-groups (long-context launches)
constexpr int kDecodeMRows = 8;      // pairs per decode tile (at most 8 of the 16 MFMA columns)
constexpr int kFp32MRows = 16;       // pairs per fp32 tile (one wave each)
constexpr int kMaxGroup = 128;       // largest q-heads-per-kv-head ratio accepted
constexpr int kBtIndexBits = 28;     // index bits in BlockEntry::bt_valid
constexpr int kMaxPoolBlocks = 1 << kBtIndexBits;

// Fixed device scratch of msa_forward_noalloc (one copy per GPU): the host
// copy of a call's packed plan, the plan as the kernels read it (block ids
// resolved), then the partial results of split tiles.
constexpr size_t kScratchPlanBytes = size_t(2) << 20;
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr size_t kScratchPartBytes = kScratchBytes - 2 * kScratchPlanBytes;

// One entry of a sequence's position-ordered block list (8 bytes).  The host
// writes the block-table index; the upload kernel replaces it, on the device,
// by the pool block id it names, so kernels never chase block_table.
struct BlockEntry {
  int32_t bt_valid;  // bits 0..27: block-table index (host) / pool block id (device);
                     // bits 28..31: valid slots - 1
  int32_t pos0;      // absolute position of slot 0
};

// One unit of kernel work: a tile of query rows of one sequence and one kv
// head, against a contiguous range of that sequence's block list.
struct WorkItem {
  int32_t kv_head;
  int32_t q_row0;    // first query row (global row index)
  int32_t n_q;       // query rows in the tile
  int32_t blk_begin; // [blk_begin, blk_end) into the block list
  int32_t blk_end;
  int32_t part_row;  // -1: final output; else first row of this split's partials
  int32_t seq;
  int32_t q_min;     // smallest query position of the tile (causal fast path)
  int32_t kind;      // kPrefill or kDecode: the work the item is (a decode item may
                     // run in the chunk kernel's launch, see Plan::items)
};

// Rows of one tile that was split over KV: n_splits partials of n_mrows rows
// each, stored back to back from part_row0.
struct MergeItem {
  int32_t kv_head;
  int32_t q_row0;
  int32_t n_q;
  int32_t part_row0;
  int32_t n_splits;
  int32_t n_mrows;
  int32_t pad0, pad1;
};

enum Kind { kPrefill = MSA_KERNEL_PREFILL, kDecode = MSA_KERNEL_DECODE,
            kFp32 = MSA_KERNEL_FP32, kMerge = MSA_KERNEL_MERGE, kUpload = MSA_KERNEL_UPLOAD,
            kWrite = MSA_KERNEL_WRITE, kNumKinds = 6 };

struct Plan {
  std::vector<BlockEntry> blocks;
  std::vector<int32_t> q_pos;
  // Per launch (prefill/chunk, decode, fp32 kernel).  When a batch holds both
  // prefill chunks and decode tokens (bf16), the decode items go into the
  // chunk kernel's launch, which runs them with the decode kernel's code: one
  // attention launch for the batch, the decode items filling compute units
  // beside the chunk items.
  std::vector<WorkItem> items[3];
  std::vector<MergeItem> merges;
  int64_t part_rows = 0;            // partial rows (each head_dim floats + 1 lse)
  int32_t max_mrows[3] = {0, 0, 0}; // largest (query row, head) count of an item, per kind
  int32_t total_q = 0;
  // Waves per work-group of the chunk launch: 4 (128-row tiles, two
  // work-groups per CU) or 8 (256-row tiles, one per CU: half the K/V
  // staging per FLOP, for launches with at least two such tiles per CU).
  int32_t chunk_waves = 4;
  // Per launch: 1 when its K/V blocks are streamed past the caches (non-
  // temporal V staging in the decode kernel): a decode launch whose K/V
  // exceeds twice the 256 MB Infinity Cache, so none of it would be found
  // there again.  Smaller launches keep V cacheable.
  int32_t stream_kv[3] = {0, 0, 0};
};

struct PlanConfig {
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t dtype = MSA_BF16;
  int32_t num_cus = 256;
  int32_t split_blocks = 0;         // >0 forces this cap on blocks per item
  int32_t chunk_waves = 0;          // 4 or 8 forces the chunk work-group size; 0: the planner's choice
};

// Checks every argument of the descriptor and builds the plan.  Host only;
// returns an MSA_* status and fills `err` on failure.
int build_plan(const msa_seg_desc* desc, const PlanConfig& cfg, Plan& plan, std::string& err);

// Kernel launch parameters (identical for every kernel kind).
struct KernelArgs {
  const void* q;
  void* out;
  float* lse;             // may be null
  const void* k;
  const void* v;
  const int32_t* block_table;
  const BlockEntry* blocks;
  const int32_t* q_pos;
  const WorkItem* items;
  const MergeItem* merges;
  float* part_o;          // [part_rows][head_dim]
  float* part_lse;        // [part_rows]
  int32_t n_items;
  int32_t n_merges;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // num_q_heads / num_kv_heads
  int32_t causal;
  float scale_log2;       // scale * log2(e)
  int32_t max_mrows;      // largest n_q * group among the launch's items
  int32_t stream_kv;      // 1: stage V with non-temporal loads (decode launches over large K/V)
  unsigned long long* trace;  // phase clocks of the chunk kernel (tracing builds only), or null
};

// KV write launch: one wave per (block-list entry, kv head).  Entry e's pos0
// holds the source row of its slot 0 (not a position).
struct WriteArgs {
  const void* k_src;      // [rows][num_kv_heads][head_dim]
  const void* v_src;
  void* k;                // pool
  void* v;
  const BlockEntry* blocks;
  int32_t n_entries;
  int32_t num_kv_heads;
};

// Device address of this GPU's copy of the fixed scratch (kScratchBytes),
// looked up once per device with that device current.  Returns an MSA_*
// status and fills `err` on failure.
int scratch_address(int device, void** ptr, std::string& err);

// Launchers (one per kernel source).  Return a hipError_t value.
int launch_prefill(const KernelArgs& a, int head_dim, int waves, void* stream);
int launch_decode(const KernelArgs& a, int head_dim, void* stream);
int launch_fp32(const KernelArgs& a, int head_dim, void* stream);
int launch_merge(const KernelArgs& a, int head_dim, int dtype, void* stream);
// row_bytes = head_dim * element size: 128, 256 or 512.
int launch_write(const WriteArgs& a, int row_bytes, void* stream);
// Copies `bytes` (a multiple of 16) of plan from device-mapped pinned host
// memory to `dst`, resolving the first `n_blocks` entries (the block list)
// through `block_table`; ids outside [0, num_blocks) are clamped into range.
int launch_upload(const void* src, void* dst, size_t bytes, int32_t n_blocks, const int32_t* block_table,
                  int32_t num_blocks, void* stream);
// With MSA_OPT_CHECK_BLOCK_IDS: counts the first n_blocks entries of the
// host-packed block list at `src` whose block-table entry is out of range
// into result[0] and keeps the smallest such block-table index in result[1]
// (device words that start at 0 and INT32_MAX).
int launch_check_ids(const void* src, int32_t n_blocks, const int32_t* block_table, int32_t num_blocks,
                     int32_t* result, void* stream);

}  // namespace msa
