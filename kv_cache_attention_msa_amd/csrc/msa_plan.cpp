// Argument checks and the split-KV work planner (host only, no HIP calls).
//
// The planner turns the caller's segment descriptors into
//  * a position-ordered block list per sequence (segments sorted by position,
//    expanded to one entry per KV block, so a 64-key kernel tile may span a
//    segment boundary and only the partially filled last block of a segment
//    wastes slots);
//  * work items: a tile of query rows of one sequence and one kv head against
//    the prefix of that sequence's block list that the tile can see (causal by
//    absolute position: a block is needed iff its first position <= the tile's
//    largest query position), cut into KV splits when the device would
//    otherwise be unevenly loaded, largest first;
//  * merge items for every tile that was split.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <limits>
#include <numeric>

#include "msa_internal.h"

namespace msa {

static int fail(std::string& err, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  err = buf;
  return code;
}

namespace {

struct Tile {
  int32_t kind, seq, q_min, q_row0, n_q, blk_begin, blk_end, nsplit;
  int32_t launch;   // the launch (kernel) that runs the tile's items
};

// Largest block-count of one work item before the planner splits a tile.
int64_t auto_chunk(int kind, int64_t total_blocks, int num_cus, int chunk_waves) {
  // Work-groups per compute unit the planner balances for: the chunk kernel
  // holds two per CU (one with 8-wave work-groups); the decode kernel holds
  // three, and two items per resident slot keep the bandwidth-bound launch
  // busy to its end (measured: 8 decode tokens over 2k-16k contexts 56.8 ->
  // 52.1 us against one item per slot, 64 tokens over 1k-8k unchanged).
  const int64_t slots_per_cu = (kind == kPrefill) ? (chunk_waves == 8 ? 1 : 2) : (kind == kDecode ? 6 : 4);
  const int64_t min_chunk = (kind == kPrefill) ? 16 : (kind == kDecode ? 32 : 4);
  const int64_t slots = std::max<int64_t>(1, slots_per_cu * num_cus);
  return std::max<int64_t>(min_chunk, (total_blocks + slots - 1) / slots);
}

// Working lists of the planner, kept per thread so that a call allocates
// nothing once they have grown.
std::vector<Tile>& plan_tiles() {
  thread_local std::vector<Tile> v;
  return v;
}
std::vector<int32_t>& plan_order() {
  thread_local std::vector<int32_t> v;
  return v;
}

// Stable sort of work items by block count, largest first.  Block counts
// are bounded by the split chunk, so a counting sort is the usual path.
void sort_by_size(std::vector<WorkItem>& v) {
  const size_t n = v.size();
  if (n < 2) return;
  int32_t mx = 0;
  for (const WorkItem& w : v) mx = std::max(mx, w.blk_end - w.blk_begin);
  if ((size_t)mx > 4 * n + 4096) {
    std::stable_sort(v.begin(), v.end(), [](const WorkItem& x, const WorkItem& y) {
      return (x.blk_end - x.blk_begin) > (y.blk_end - y.blk_begin);
    });
    return;
  }
  thread_local std::vector<int32_t> start;
  thread_local std::vector<WorkItem> tmp;
  start.assign((size_t)mx + 2, 0);
  for (const WorkItem& w : v) ++start[(size_t)(mx - (w.blk_end - w.blk_begin)) + 1];
  for (size_t i = 1; i < start.size(); ++i) start[i] += start[i - 1];
  tmp.resize(n);
  for (const WorkItem& w : v) tmp[(size_t)start[(size_t)(mx - (w.blk_end - w.blk_begin))]++] = w;
  v.swap(tmp);
}

}  // namespace

int build_plan(const msa_seg_desc* d, const PlanConfig& cfg, Plan& plan, std::string& err) {
  const int INV = MSA_ERR_INVALID_ARG, UNS = MSA_ERR_UNSUPPORTED;
  plan.q_pos.clear();
  for (auto& v : plan.items) v.clear();
  plan.merges.clear();
  plan.part_rows = 0;
  plan.total_q = 0;
  for (auto& x : plan.max_mrows) x = 0;

  if (!d) return fail(err, INV, "seg_desc is NULL");
  if (cfg.head_dim != 64 && cfg.head_dim != 128)
    return fail(err, UNS, "head_dim %d is not supported (64 or 128)", cfg.head_dim);
  if (cfg.dtype != MSA_BF16 && cfg.dtype != MSA_FP32)
    return fail(err, UNS, "dtype %d is not supported", cfg.dtype);
  if (cfg.num_kv_heads <= 0) return fail(err, INV, "num_kv_heads must be > 0");
  if (d->batch < 0) return fail(err, INV, "batch %d < 0", d->batch);
  if (d->num_q_heads <= 0) return fail(err, INV, "num_q_heads %d <= 0", d->num_q_heads);
  if (d->num_q_heads % cfg.num_kv_heads != 0)
    return fail(err, INV, "num_q_heads %d is not a multiple of num_kv_heads %d", d->num_q_heads,
                cfg.num_kv_heads);
  const int group = d->num_q_heads / cfg.num_kv_heads;
  if (group > kMaxGroup) return fail(err, UNS, "GQA ratio %d exceeds %d", group, kMaxGroup);
  if (d->causal != 0 && d->causal != 1) return fail(err, INV, "causal must be 0 or 1");
  if (!std::isfinite(d->scale) || d->scale < 0.f)
    return fail(err, INV, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  if (d->block_table_len < 0) return fail(err, INV, "block_table_len < 0");
  if (d->block_table_len > (1 << kBtIndexBits))
    return fail(err, MSA_ERR_WORKSPACE, "block_table_len %d exceeds 2^%d", d->block_table_len,
                kBtIndexBits);
  const int B = d->batch;
  if (B == 0) {
    plan.blocks.clear();
    return MSA_OK;
  }
  if (!d->q_offsets || !d->seg_offsets) return fail(err, INV, "q_offsets or seg_offsets is NULL");
  if (d->q_offsets[0] != 0 || d->seg_offsets[0] != 0)
    return fail(err, INV, "q_offsets[0] and seg_offsets[0] must be 0");
  for (int b = 0; b < B; ++b) {
    if (d->q_offsets[b + 1] < d->q_offsets[b])
      return fail(err, INV, "q_offsets decreases at sequence %d", b);
    if (d->seg_offsets[b + 1] < d->seg_offsets[b])
      return fail(err, INV, "seg_offsets decreases at sequence %d", b);
  }
  const int32_t total_q = d->q_offsets[B];
  const int32_t total_segs = d->seg_offsets[B];
  if ((int64_t)total_q * d->num_q_heads > std::numeric_limits<int32_t>::max())
    return fail(err, MSA_ERR_WORKSPACE, "total_q * num_q_heads exceeds 2^31");
  if (total_q > 0 && !d->q_pos) return fail(err, INV, "q_pos is NULL");
  if (total_segs > 0 && !d->segs) return fail(err, INV, "segs is NULL");
  plan.total_q = total_q;

  // Segments: checks, and the number of blocks they cover in all.
  int64_t n_blocks = 0;
  for (int32_t s = 0; s < total_segs; ++s) {
    const msa_segment& sg = d->segs[s];
    if (sg.len < 0 || sg.pos_start < 0 || sg.bt_start < 0)
      return fail(err, INV, "segment %d: negative pos_start, len or bt_start", s);
    if ((int64_t)sg.pos_start + sg.len > std::numeric_limits<int32_t>::max())
      return fail(err, INV, "segment %d: pos_start + len overflows int32", s);
    const int64_t nblk = (sg.len + kBlock - 1) / kBlock;
    if ((int64_t)sg.bt_start + nblk > d->block_table_len)
      return fail(err, INV, "segment %d: blocks [%d, %lld) exceed block_table_len %d", s, sg.bt_start,
                  (long long)(sg.bt_start + nblk), d->block_table_len);
    n_blocks += nblk;
  }
  if (n_blocks > std::numeric_limits<int32_t>::max() / 2)
    return fail(err, MSA_ERR_WORKSPACE, "%lld blocks in one call exceed 2^30", (long long)n_blocks);
  // resize() keeps the entries of an earlier call; every one is rewritten below
  plan.blocks.resize((size_t)n_blocks);

  // Chunk work-group size: 8 waves (256-row tiles, one work-group per CU)
  // for a batch of prefill chunks only, whose 256-row tiles number at least
  // two per compute unit and whose contexts average at least 8 MiB of K/V per
  // kv head (twice an XCD's L2): each K/V block is then staged into half as
  // many work-groups, and those re-reads would otherwise go past the L2 (the
  // heavy-fragmentation workload, 2 x 32k context: 1.97 -> 1.92 ms).  Else 4
  // waves (128-row tiles, two per CU): shorter contexts stay in the L2, and
  // a decode item would leave half of an 8-wave work-group idle (both measured
  // slower with 8 waves).
  plan.chunk_waves = 4;
  if (cfg.dtype == MSA_BF16) {
    const int32_t wide_rows = std::max(1, kPrefillMRowsWide / group);
    int64_t wide_tiles = 0, tile_blocks = 0;
    bool any_decode_seq = false;
    for (int b = 0; b < B; ++b) {
      const int32_t nq = d->q_offsets[b + 1] - d->q_offsets[b];
      if (nq == 0) continue;
      if (group <= kDecodeMRows && (int64_t)nq * group <= kDecodeMRows) {
        any_decode_seq = true;
        continue;
      }
      int64_t nblk = 0;
      for (int32_t sg = d->seg_offsets[b]; sg < d->seg_offsets[b + 1]; ++sg) nblk += (d->segs[sg].len + kBlock - 1) / kBlock;
      const int64_t t = (nq + wide_rows - 1) / wide_rows;
      wide_tiles += t;
      tile_blocks += t * nblk;
    }
    const int64_t block_bytes = (int64_t)kBlock * cfg.head_dim * 2 * 2;   // K and V of one block, one kv head
    if (!any_decode_seq && wide_tiles * cfg.num_kv_heads >= 2 * (int64_t)cfg.num_cus &&
        tile_blocks * block_bytes >= wide_tiles * (int64_t(8) << 20))
      plan.chunk_waves = 8;
    if (cfg.chunk_waves == 4 || cfg.chunk_waves == 8) plan.chunk_waves = cfg.chunk_waves;
  }

  std::vector<Tile>& tiles = plan_tiles();
  std::vector<int32_t>& order = plan_order();
  tiles.clear();
  int32_t cursor = 0;
  for (int b = 0; b < B; ++b) {
    const int32_t s0 = d->seg_offsets[b], s1 = d->seg_offsets[b + 1];
    // Segments in position order; callers usually pass them so already.
    bool sorted = true;
    for (int32_t s = s0 + 1; s < s1 && sorted; ++s) sorted = d->segs[s - 1].pos_start <= d->segs[s].pos_start;
    order.clear();
    for (int32_t s = s0; s < s1; ++s)
      if (d->segs[s].len > 0) order.push_back(s);
    if (!sorted)
      std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
        return d->segs[x].pos_start < d->segs[y].pos_start;
      });
    for (size_t i = 1; i < order.size(); ++i) {
      const msa_segment& p = d->segs[order[i - 1]];
      const msa_segment& c = d->segs[order[i]];
      if ((int64_t)p.pos_start + p.len > c.pos_start)
        return fail(err, INV, "sequence %d: segments %d and %d overlap in position", b, order[i - 1],
                    order[i]);
    }
    const int32_t seq_blk0 = cursor;
    BlockEntry* dst = plan.blocks.data();
    for (int32_t s : order) {
      // locals, so that the stores below need not reload the segment
      const int32_t len = d->segs[s].len, pos = d->segs[s].pos_start, bt = d->segs[s].bt_start;
      const int32_t full = len / kBlock, tail = len - full * kBlock;
      const uint32_t full_tag = (uint32_t)(kBlock - 1) << kBtIndexBits;
      BlockEntry* out = dst + cursor;
      int32_t tag = (int32_t)((uint32_t)bt | full_tag), p0 = pos;
      for (int32_t j = 0; j < full; ++j, ++tag, p0 += kBlock) {
        out[j].bt_valid = tag;
        out[j].pos0 = p0;
      }
      cursor += full;
      if (tail)
        dst[cursor++] = BlockEntry{(int32_t)((uint32_t)(bt + full) | ((uint32_t)(tail - 1) << kBtIndexBits)),
                                   pos + full * kBlock};
    }
    const int32_t seq_blk1 = cursor;

    // Query tiles of this sequence.
    const int32_t q0 = d->q_offsets[b], q1 = d->q_offsets[b + 1];
    const int32_t nq = q1 - q0;
    if (nq == 0) continue;
    int kind;
    int32_t tile_rows;
    if (cfg.dtype == MSA_FP32) {
      kind = kFp32;
      tile_rows = std::max(1, kFp32MRows / group);
    } else if (group <= kDecodeMRows && (int64_t)nq * group <= kDecodeMRows) {
      kind = kDecode;
      tile_rows = nq;
    } else {
      kind = kPrefill;
      tile_rows = std::max(1, (plan.chunk_waves == 8 ? kPrefillMRowsWide : kPrefillMRows) / group);
    }
    for (int32_t r = q0; r < q1; r += tile_rows) {
      const int32_t n = std::min(tile_rows, q1 - r);
      int32_t end = seq_blk1;
      int32_t qmin = d->q_pos[r], qmax = d->q_pos[r];
      for (int32_t i = r + 1; i < r + n; ++i) {
        qmin = std::min(qmin, d->q_pos[i]);
        qmax = std::max(qmax, d->q_pos[i]);
      }
      if (d->causal) {
        // first block whose slot-0 position is beyond every query of the tile
        auto it = std::upper_bound(plan.blocks.begin() + seq_blk0, plan.blocks.begin() + seq_blk1, qmax,
                                   [](int32_t v, const BlockEntry& e) { return v < e.pos0; });
        end = (int32_t)(it - plan.blocks.begin());
      }
      tiles.push_back(Tile{kind, b, qmin, r, n, seq_blk0, end, 1, kind});
    }
  }
  plan.q_pos.assign(d->q_pos, d->q_pos + total_q);

  // A batch of prefill chunks and decode tokens runs in one launch: the
  // decode tiles join the chunk kernel's items (it runs them with the decode
  // code), balanced together with them.
  bool any_prefill = false, any_decode = false;
  for (const Tile& t : tiles) {
    any_prefill |= t.kind == kPrefill;
    any_decode |= t.kind == kDecode;
  }
  if (any_prefill && any_decode)
    for (Tile& t : tiles) t.launch = kPrefill;

  // Expand tiles over kv heads and split long ones.
  int64_t total_blocks[3] = {0, 0, 0};
  for (const Tile& t : tiles) total_blocks[t.launch] += (int64_t)(t.blk_end - t.blk_begin) * cfg.num_kv_heads;
  {
    // K and V of one block and kv head; a launch streams its K/V past the
    // caches when it reads more than twice the Infinity Cache (measured on
    // 64 decode tokens over 1k-8k contexts, 1.28 GB: 212 -> 203 us; 8 tokens
    // over 2k-16k, 0.32 GB, read 10 % slower with streamed V, their V partly
    // still cached from the previous call).
    const int64_t block_bytes = (int64_t)kBlock * cfg.head_dim * 2 * (cfg.dtype == MSA_FP32 ? 4 : 2);
    for (int k = 0; k < 3; ++k) plan.stream_kv[k] = 0;
    plan.stream_kv[kDecode] = total_blocks[kDecode] * block_bytes > (int64_t(512) << 20) ? 1 : 0;
  }
  int64_t chunk[3];
  for (int k = 0; k < 3; ++k)
    chunk[k] = cfg.split_blocks > 0 ? cfg.split_blocks : auto_chunk(k, total_blocks[k], cfg.num_cus, plan.chunk_waves);

  // Split count of every tile, then the item and merge counts, so that the
  // lists are sized once and written in place.
  size_t n_items[3] = {0, 0, 0}, n_merges = 0;
  int64_t part_rows = 0;
  for (Tile& t : tiles) {
    const int32_t nblk = t.blk_end - t.blk_begin;
    const int64_t c = chunk[t.launch];
    int32_t nsplit = 1;
    if (cfg.split_blocks > 0 ? nblk > c : nblk > c + c / 2) nsplit = (int32_t)((nblk + c - 1) / c);
    const int32_t align = (t.kind == kPrefill) ? 4 : 1;  // prefill consumes 4 blocks per step
    nsplit = std::max(1, std::min(nsplit, (nblk + align - 1) / align));
    t.nsplit = nsplit;
    const int32_t n_mrows = t.n_q * group;
    plan.max_mrows[t.launch] = std::max(plan.max_mrows[t.launch], n_mrows);
    n_items[t.launch] += (size_t)nsplit * cfg.num_kv_heads;
    if (nsplit > 1) {
      n_merges += cfg.num_kv_heads;
      part_rows += (int64_t)nsplit * n_mrows * cfg.num_kv_heads;
    }
  }
  if (part_rows > std::numeric_limits<int32_t>::max())
    return fail(err, MSA_ERR_WORKSPACE, "split partials exceed 2^31 rows");
  for (int k = 0; k < 3; ++k) plan.items[k].resize(n_items[k]);
  plan.merges.resize(n_merges);
  WorkItem* item_out[3] = {plan.items[0].data(), plan.items[1].data(), plan.items[2].data()};
  MergeItem* merge_out = plan.merges.data();
  std::vector<int32_t>& bounds = plan_order();  // reused: split boundaries of one tile
  int32_t part = 0;
  for (const Tile& t : tiles) {
    WorkItem*& wo = item_out[t.launch];
    if (t.nsplit == 1) {
      for (int32_t h = 0; h < cfg.num_kv_heads; ++h)
        *wo++ = WorkItem{h, t.q_row0, t.n_q, t.blk_begin, t.blk_end, -1, t.seq, t.q_min, t.kind};
      continue;
    }
    // the same block ranges for every kv head
    const int32_t nblk = t.blk_end - t.blk_begin;
    const int32_t align = (t.kind == kPrefill) ? 4 : 1;
    const int32_t units = (nblk + align - 1) / align;
    bounds.resize((size_t)t.nsplit + 1);
    bounds[0] = 0;
    for (int32_t s = 0; s < t.nsplit; ++s)
      bounds[s + 1] = std::min(nblk, (int32_t)((int64_t)units * (s + 1) / t.nsplit) * align);
    const int32_t n_mrows = t.n_q * group;
    for (int32_t h = 0; h < cfg.num_kv_heads; ++h) {
      for (int32_t s = 0; s < t.nsplit; ++s)
        *wo++ = WorkItem{h, t.q_row0, t.n_q, t.blk_begin + bounds[s], t.blk_begin + bounds[s + 1],
                         part + s * n_mrows, t.seq, t.q_min, t.kind};
      *merge_out++ = MergeItem{h, t.q_row0, t.n_q, part, t.nsplit, n_mrows, 0, 0};
      part += t.nsplit * n_mrows;
    }
  }
  plan.part_rows = part;
  // Largest work first, so the tail of the launch is made of small items;
  // items of equal size keep their order.
  for (auto& v : plan.items) sort_by_size(v);
  return MSA_OK;
}

}  // namespace msa
