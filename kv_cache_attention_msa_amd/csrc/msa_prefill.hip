// Chunk (prefill) kernel for bf16 pools: exact softmax attention of a tile of
// 128 or 256 (query row, q head) pairs against a run of KV blocks, with both
// matrix products on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulate).
//
// Work-group: W = 4 waves (two work-groups per CU) or W = 8 (one per CU, for
// launches with enough tiles: each K/V block is staged into half as many
// work-groups); wave w owns tile rows 32w..32w+31.  A tile row is a (query
// row, head of the kv head's GQA group) pair, so the K/V tile staged in LDS
// serves every q head of the group.
//
// Per step of 64 keys (4 pool blocks of the position-ordered block list, which
// may span segment boundaries):
//   * S^T = K Q^T (K from LDS, Q^T resident in registers), so each lane holds
//     one tile row's scores for 16 keys;
//   * then the next step's K and V go from the pool straight into the other
//     LDS tile by LDS DMA (buffer loads with the lds flag, one buffer
//     resource per pool block, whose 4 KiB per kv head are contiguous; each
//     wave moves one block, or with 8 waves the K or the V of one), so staging
//     costs the waves neither registers nor LDS writes, and has the rest of
//     the step to land;
//   * keys outside a block's valid slots, past the item's blocks, or (causal)
//     at a position after the row's query position get score -inf by select;
//     steps that are entirely visible to every row skip the mask;
//   * online softmax in the exp2 domain (scale * log2 e folded into one FMA)
//     against a per-row reference that moves only when needed;
//   * P is rounded to bf16 in place of the S accumulator registers and used as
//     the B operand of O^T += V^T P^T, whose V^T operand comes from the
//     row-major V tile through the transposing LDS read of gfx950.
// Each block's buffer resource covers only its valid slots: DMA reads past
// them return zero, so slots that hold no key are zero in LDS and the
// 0-probabilities never meet pool contents (NaN * 0 would poison the row).
//
// The launch may also hold decode items (the decode tokens of a batch that
// mixes them with prefill chunks): a work-group given one runs the decode
// kernel's code (msa_decode_item.h) in this kernel's LDS, so the whole batch
// is one launch and the bandwidth-bound decode items share the chip with the
// MFMA-bound chunk items.
#include "msa_common.h"
#include "msa_decode_item.h"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kStepKeys = 64;   // keys per step = 4 blocks
constexpr float kRefSumLimit = 1048576.f;  // 2^20: largest accepted partial row sum per step

// LDS tiles, one per buffer (two separate LDS variables, so that the
// compiler can tell reads of one from DMA writes into the other).  Both K
// and V are stored row-major (one key per row) with their 16-byte chunks
// XOR-swizzled, and are filled by LDS DMA straight from the pool.
template <int D>
struct StepTile {
  uint4 k[kStepKeys][D / 8];   // [key][chunk]: K rows, chunk c at c ^ k_swz(key)
  uint4 v[kStepKeys][D / 8];   // [key][chunk]: V rows, chunk c at c ^ v_swz(key)
};

// K operand reads take 32 consecutive rows at one chunk index: with the row
// XOR the 16-byte reads of a wave spread over all banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}
// V operand reads (ds_read_b64_tr_b16) take, per half-wave, 64 bytes (32
// head_dim values) of 4 consecutive rows; the XOR moves each of the 4 rows
// to its own quarter of the banks.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  if constexpr (D == 128) return (row & 3) << 2;
  else return (row & 2) << 1;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// K operands of rows `row` and `row + 32` at chunk c: both rows have the same
// swizzle (it depends on row % 16), so one address serves both.
template <int D>
__device__ __forceinline__ void ld_k2(const StepTile<D>& tl, int row, int c, bf16x8& k0, bf16x8& k1) {
  const uint4* p = &tl.k[row][c ^ k_swz<D>(row)];
  k0 = as_bf16x8(p[0]);
  k1 = as_bf16x8(p[32 * (D / 8)]);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, component r of lane i's result is 16-bit element i % 4 of the 8
// bytes addressed by lane 4r + i / 4 of the group.
__device__ __forceinline__ s16x4 ld_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<char*>(p)));
}

// Descriptors of one step's (up to) 4 blocks.  Plain scalar fields rather
// than arrays, so that no private array is ever indexed at run time.
struct StepMeta {
  int nb;                          // blocks in this step (1..4)
  int ph0, ph1, ph2, ph3;          // pool block ids (always valid ids)
  int ps0, ps1, ps2, ps3;          // positions of slot 0
  int vl0, vl1, vl2, vl3;          // valid slots (0 past the item's end)
  bool full;                       // 64 keys, all visible to every row of the tile
  __device__ __forceinline__ int phys(int b) const { return b == 0 ? ph0 : b == 1 ? ph1 : b == 2 ? ph2 : ph3; }
  __device__ __forceinline__ int pos0(int b) const { return b == 0 ? ps0 : b == 1 ? ps1 : b == 2 ? ps2 : ps3; }
  __device__ __forceinline__ int valid(int b) const { return b == 0 ? vl0 : b == 1 ? vl1 : b == 2 ? vl2 : vl3; }
};

// The block list is padded with 4 spare entries and indices are clamped to
// them, so the entries of any step (also one past the item's last) are
// readable; entries past the item's end get valid = 0 (their ids are still
// pool block ids).
__device__ __forceinline__ void load_meta(const KernelArgs& a, int blk, int blk_end, int q_min, StepMeta& m) {
  m.nb = max(0, min(4, blk_end - blk));
  const int last = blk_end + 3;
  const BlockEntry e0 = a.blocks[min(blk, last)], e1 = a.blocks[min(blk + 1, last)];
  const BlockEntry e2 = a.blocks[min(blk + 2, last)], e3 = a.blocks[min(blk + 3, last)];
  m.ph0 = entry_block(e0); m.ph1 = entry_block(e1); m.ph2 = entry_block(e2); m.ph3 = entry_block(e3);
  m.ps0 = e0.pos0; m.ps1 = e1.pos0; m.ps2 = e2.pos0; m.ps3 = e3.pos0;
  m.vl0 = m.nb > 0 ? entry_valid(e0) : 0;
  m.vl1 = m.nb > 1 ? entry_valid(e1) : 0;
  m.vl2 = m.nb > 2 ? entry_valid(e2) : 0;
  m.vl3 = m.nb > 3 ? entry_valid(e3) : 0;
  m.full = m.nb == 4 && m.vl0 == 16 && m.vl1 == 16 && m.vl2 == 16 && m.vl3 == 16 &&
           (!a.causal || m.ps3 + 15 <= q_min);
}

// The valid rows of one pool block of one kv head as a buffer resource:
// loads past them (slots without a key, whole blocks past the item's end)
// read zero, so no pool contents outside the keys reach LDS.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* pool, int kv_head, int num_kv_heads, int phys,
                                                             int valid) {
  const char* p = (const char*)pool + ((int64_t)phys * num_kv_heads + kv_head) * (kBlock * D * 2);
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, valid * D * 2, 0x00020000);
}

// Per-lane byte offsets (inside a pool block) of the 16-byte chunks that the
// DMA of one step brings in.  One DMA instruction fills 1 KiB of LDS, lane j
// at byte 16 j, i.e. (D = 128) row 4i + j/16 of the block, physical chunk
// j % 16; the lane fetches the logical chunk that belongs there.
template <int D>
struct DmaOffsets {
  uint32_t k[D / 32];
  uint32_t v;               // + i KiB for instruction i
};
template <int D>
__device__ __forceinline__ DmaOffsets<D> dma_offsets(int lane) {
  constexpr int CPR = D / 8;      // chunks per row
  constexpr int RPI = 64 / CPR;   // rows per instruction
  DmaOffsets<D> o;
  const int p = lane % CPR, r = lane / CPR;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int row = i * RPI + r;  // row inside the block (the block's base row is a multiple of 16)
    o.k[i] = (uint32_t)(row * CPR + (p ^ k_swz<D>(row))) * 16u;
  }
  o.v = (uint32_t)(r * CPR + (p ^ v_swz<D>(r))) * 16u;  // v_swz depends on row % 4 only
  return o;
}

// One step's K and V from the pool into a tile by LDS DMA: with 4 waves,
// wave w moves K and V of block w; with 8, waves 0-3 move K and waves 4-7 V of
// block w % 4.
template <int D, int W>
__device__ __forceinline__ void dma_step(const KernelArgs& a, int kv_head, const StepMeta& m, StepTile<D>& tl,
                                         int wave, const DmaOffsets<D>& o) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  const int b = wave & 3;
  const int phys = m.phys(b), valid = m.valid(b);
  if (W == 4 || wave < 4) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(a.k, kv_head, a.num_kv_heads, phys, valid);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int off = (int)o.k[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)&tl.k[16 * b + i * RPI][0], 16, off, 0, 0, 0);
    }
  }
  if (W == 4 || wave >= 4) {
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(a.v, kv_head, a.num_kv_heads, phys, valid);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int off = (int)o.v + i * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)&tl.v[16 * b + i * RPI][0], 16, off, 0, 0, 0);
    }
  }
}

// Scores of one 32-row half for a step: s{kb} register r holds key
// 32kb + 8(r/4) + 4h + r%4 (block 2kb + r/8, slot 8((r/4)&1) + 4h + r%4).
// Within a block, positions run with the slot, so a key of block b is
// visible to the row iff its slot is below lim(b) = min(valid(b),
// qpos - pos0(b) + 1) (valid(b) when not causal): one compare per score.
__device__ __forceinline__ int block_lim(const StepMeta& m, int b, int qpos, bool causal) {
  const int v = m.valid(b);
  return causal ? min(v, qpos - m.pos0(b) + 1) : v;
}

__device__ __forceinline__ void mask_half(f32x16& s0, f32x16& s1, const StepMeta& m, int h, int qpos, bool causal) {
  const int l0 = block_lim(m, 0, qpos, causal), l1 = block_lim(m, 1, qpos, causal);
  const int l2 = block_lim(m, 2, qpos, causal), l3 = block_lim(m, 3, qpos, causal);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int slot = 8 * ((r >> 2) & 1) + 4 * h + (r & 3);
    s0[r] = slot < ((r >> 3) ? l1 : l0) ? s0[r] : kNegInf;
    s1[r] = slot < ((r >> 3) ? l3 : l2) ? s1[r] : kNegInf;
  }
}

__device__ __forceinline__ float row_max(const f32x16& s0, const f32x16& s1) {
  float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    m0 = __builtin_fmaxf(m0, __builtin_fmaxf(s0[r], s0[r + 1]));
    m1 = __builtin_fmaxf(m1, __builtin_fmaxf(s1[r], s1[r + 1]));
  }
  const float mx = fmaxf(m0, m1);
  return fmaxf(mx, __shfl_xor(mx, 32, 64));
}

// p = exp2(s * c2 - mu) rounded to bf16 in pw (word j of kb: regs 2j, 2j+1);
// returns this lane's part of the row sum (the other lane half holds the
// rest), summed from the rounded p that the PV product uses, two at a time
// (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float exp_half(const f32x16& s0, const f32x16& s1, float c2, float mu, uint32_t (&pw)[16]) {
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, -mu));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s0[r + 1], c2, -mu));
    const float p2 = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, -mu));
    const float p3 = __builtin_amdgcn_exp2f(fmaf(s1[r + 1], c2, -mu));
    pw[r / 2] = pack_bf16x2(p0, p1);
    pw[8 + r / 2] = pack_bf16x2(p2, p3);
  }
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float ra = 0.f, rb = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    ra = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[j]), one, ra, false);
    rb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[j + 1]), one, rb, false);
  }
  return ra + rb;
}

struct RowInfo {
  bool ok;
  int token, head, qpos;
};

__device__ __forceinline__ RowInfo row_info(const KernelArgs& a, const WorkItem& it, int mrow) {
  RowInfo ri;
  const int g = a.group;
  ri.ok = mrow < it.n_q * g;
  ri.token = it.q_row0 + (ri.ok ? mrow / g : 0);
  ri.head = it.kv_head * g + (ri.ok ? mrow % g : 0);
  ri.qpos = ri.ok ? a.q_pos[ri.token] : INT_MIN;
  return ri;
}

template <int D>
__device__ __forceinline__ void write_rows(const KernelArgs& a, const WorkItem& it, const RowInfo& ri, int mrow, int h,
                                           const f32x16 (&acc)[D / 32], float m, float l_tot) {
  if (!ri.ok) return;
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m + log2f(l_tot)) * kLn2 : kNegInf;
  if (it.part_row < 0) {
    bf16_t* orow = (bf16_t*)a.out + ((int64_t)ri.token * a.num_q_heads + ri.head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + q4 * 8 + h * 4;
        uint2 w;
        w.x = pack_bf16x2(acc[db][q4 * 4 + 0] * inv, acc[db][q4 * 4 + 1] * inv);
        w.y = pack_bf16x2(acc[db][q4 * 4 + 2] * inv, acc[db][q4 * 4 + 3] * inv);
        *(uint2*)(orow + d0) = w;
      }
    if (a.lse && h == 0) a.lse[(int64_t)ri.token * a.num_q_heads + ri.head] = lse_v;
  } else {
    float* prow = a.part_o + (int64_t)(it.part_row + mrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + q4 * 8 + h * 4;
        *(float4*)(prow + d0) = make_float4(acc[db][q4 * 4] * inv, acc[db][q4 * 4 + 1] * inv,
                                            acc[db][q4 * 4 + 2] * inv, acc[db][q4 * 4 + 3] * inv);
      }
    if (h == 0) a.part_lse[it.part_row + mrow] = lse_v;
  }
}

// Per-lane byte offset, inside a tile's V rows, of the 8 bytes this lane
// addresses for the V^T operand of head_dim block db (rows 16 ks (+8) are
// added as immediates).  Lane L addresses row 4 (L / 32) + (L / 4) % 4 and
// head_dim values 32 db + 16 ((L / 16) % 2) + 4 (L % 4) .. +4; after the
// transposing read lane L holds, for d = 32 db + L % 32, the keys
// 4 (L / 32) + 0..3 (first read) and 8 + 4 (L / 32) + 0..3 (second read) —
// the keys whose probabilities the lane holds in P (see exp_half).
template <int D>
__device__ __forceinline__ uint32_t vtr_offset(int lane, int db) {
  const int rr = (lane >> 2) & 3;
  const int row = 4 * (lane >> 5) + rr;
  const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
  return (uint32_t)(row * 2 * D + ((chunk ^ v_swz<D>(rr)) << 4) + 8 * (lane & 1));
}

// Per-tile state of a lane across steps.
template <int D>
struct TileState {
  bf16x8 qop[D / 16];     // Q^T operand: q[row][16ks + 8h .. +8) for every ks
  f32x16 acc[D / 32];     // O^T accumulators
  float m, l;             // per-row reference (log2 domain) and partial row sum
};

// Phase clocks (measurement builds with MSA_PHASE_TRACE only): the shader
// clock (s_memtime) is read between scheduling fences at the phase boundaries
// of every step -- QK product issued, DMA issued, mask, softmax, PV product
// issued, metadata + barrier -- and summed per phase and wave.  Reading the
// clock waits for it, so a traced step runs somewhat longer than a plain one.
#ifdef MSA_PHASE_TRACE
struct PhaseClock {
  unsigned long long last = 0, begin = 0;
  unsigned long long sum[6] = {0, 0, 0, 0, 0, 0};
  unsigned long long steps = 0;
};
__device__ __forceinline__ unsigned long long clock_now() {
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);
  return t;
}
#define PHASE_START(pc) ((pc).last = clock_now())
#define PHASE_MARK(pc, k)                             \
  do {                                                \
    const unsigned long long t_ = clock_now();        \
    (pc).sum[k] += t_ - (pc).last;                    \
    (pc).last = t_;                                   \
  } while (0)
#else
struct PhaseClock {};
#define PHASE_START(pc) ((void)(pc))
#define PHASE_MARK(pc, k) ((void)(pc))
#endif

// One step of 64 keys on tile `tl`; the next step's K and V go into `nx` by
// DMA meanwhile.  Ends with this wave's DMA complete and a work-group barrier.
template <int D, int W>
__device__ __forceinline__ void chunk_step(const KernelArgs& a, const WorkItem& it, const RowInfo& ri, TileState<D>& st,
                                           const StepTile<D>& tl, StepTile<D>& nx, StepMeta& cur, StepMeta& nxt,
                                           int next_blk, int wave, int lane, const DmaOffsets<D>& dof,
                                           const uint32_t (&voff)[D / 32], PhaseClock& pc) {
  const int h = lane >> 5;
  const int col = lane & 31;
  const float c2 = a.scale_log2;

  PHASE_START(pc);
  // the compiler's interleaving of LDS reads with MFMAs (IGLP strategy 0)
  // for the step: measured 0.3-1.2 % faster than its default schedule
  __builtin_amdgcn_iglp_opt(0);
  // ---- S^T = K Q^T for 64 keys ----
  f32x16 s0 = (f32x16){0}, s1 = (f32x16){0};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    bf16x8 k0, k1;
    ld_k2<D>(tl, col, 2 * ks + h, k0, k1);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, st.qop[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, st.qop[ks], s1, 0, 0, 0);
  }
  PHASE_MARK(pc, 0);

  dma_step<D, W>(a, it.kv_head, nxt, nx, wave, dof);
  PHASE_MARK(pc, 1);
  if (!cur.full) mask_half(s0, s1, cur, h, ri.qpos, a.causal);
  PHASE_MARK(pc, 2);

  // ---- online softmax (exp2 domain) ----
  // Probabilities are taken against a per-row reference m instead of the
  // exact running max: exact all the same, since output and row sum share
  // the reference.  The reference only has to keep exp2 in range, so the
  // row max is computed only when a lane's partial row sum leaves
  // [0, 2^20] (some p > 2^15) or the row has no reference yet; then rows
  // whose max exceeds m by more than 2^8 move m to it, rescale their
  // accumulators and recompute p.  In steady state a step costs no max
  // and no rescale.
  uint32_t pw[16];
  float rs = exp_half(s0, s1, c2, st.m == kNegInf ? 0.f : st.m, pw);
  if (__builtin_amdgcn_ballot_w64(st.m == kNegInf || !(rs <= kRefSumLimit))) {
    const float mx = row_max(s0, s1) * c2;
    const bool grow = mx != kNegInf && (st.m == kNegInf || mx > st.m + 8.f);
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - mx) : 1.f;  // m = -inf: 0
    st.m = grow ? mx : st.m;
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.acc[i] *= alpha;
    rs = exp_half(s0, s1, c2, st.m == kNegInf ? 0.f : st.m, pw);
  }
  st.l += rs;
  PHASE_MARK(pc, 3);

  // ---- O^T += V^T P^T ----
  const char* vb = (const char*)&tl.v[0][0];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int w0 = (ks >> 1) * 8 + (ks & 1) * 4;
    const bf16x8 pop = as_bf16x8(make_uint4(pw[w0], pw[w0 + 1], pw[w0 + 2], pw[w0 + 3]));
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const char* p = vb + voff[db] + ks * 16 * 2 * D;
      const s16x4 lo = ld_tr(p), hi = ld_tr(p + 8 * 2 * D);
      const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pop, st.acc[db], 0, 0, 0);
    }
  }
  PHASE_MARK(pc, 4);

  cur = nxt;
  load_meta(a, next_blk, it.blk_end, it.q_min, nxt);
  __syncthreads();   // waits for this wave's DMA, then for every wave
  PHASE_MARK(pc, 5);
#ifdef MSA_PHASE_TRACE
  pc.steps += 1;
#endif
}

template <int D, int W>
__global__ __launch_bounds__(64 * W, 2) void msa_prefill_kernel(KernelArgs a) {
  __shared__ StepTile<D> tile0;
  __shared__ StepTile<D> tile1;
  const WorkItem it = a.items[blockIdx.x];
  if (it.kind == kDecode) {
    static_assert(sizeof(dec::VRing<D>) <= sizeof(StepTile<D>), "decode buffers must fit in a tile");
    // the decode code runs on 4 waves; the others of an 8-wave work-group
    // only take part in its barriers
    if (W == 8 && threadIdx.x >= dec::kDecodeThreads) {
      dec::decode_item_idle();
      return;
    }
    dec::VRing<D>& vr0 = *reinterpret_cast<dec::VRing<D>*>(&tile0);
    dec::VRing<D>& vr1 = *reinterpret_cast<dec::VRing<D>*>(&tile1);
    if (it.n_q * a.group <= 4)
      dec::decode_item<D, 4>(a, it, vr0, vr1);
    else
      dec::decode_item<D, 8>(a, it, vr0, vr1);
    return;
  }
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int h = lane >> 5;        // lane half: which 8 of each 16 reduction indices
  const int col = lane & 31;      // tile row within the wave
  const int mrow = wave * 32 + col;
  const RowInfo ri = row_info(a, it, mrow);

  TileState<D> st;
  {
    // Q^T operand: lane holds q[row][16ks + 8h .. +8) for every ks.
    const bf16_t* qrow = (const bf16_t*)a.q + ((int64_t)ri.token * a.num_q_heads + ri.head) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      st.qop[ks] = as_bf16x8(ri.ok ? *(const uint4*)(qrow + ks * 16 + h * 8) : make_uint4(0, 0, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < D / 32; ++i) st.acc[i] = (f32x16){0};
  st.m = kNegInf;
  st.l = 0.f;

  const int nblk = it.blk_end - it.blk_begin;
  const int nsteps = (nblk + 3) >> 2;
  if (nsteps > 0) {
    const DmaOffsets<D> dof = dma_offsets<D>(lane);
    uint32_t voff[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) voff[db] = vtr_offset<D>(lane, db);
    PhaseClock pc;
#ifdef MSA_PHASE_TRACE
    pc.begin = clock_now();
#endif
    StepMeta cur, nxt;
    load_meta(a, it.blk_begin, it.blk_end, it.q_min, cur);
    dma_step<D, W>(a, it.kv_head, cur, tile0, wave, dof);
    load_meta(a, it.blk_begin + 4, it.blk_end, it.q_min, nxt);
    __syncthreads();

    // Unrolled by two so that each step's tiles are known at compile time.
    for (int s = 0; s < nsteps; s += 2) {
      chunk_step<D, W>(a, it, ri, st, tile0, tile1, cur, nxt, it.blk_begin + 4 * (s + 2), wave, lane, dof, voff, pc);
      if (s + 1 >= nsteps) break;
      chunk_step<D, W>(a, it, ri, st, tile1, tile0, cur, nxt, it.blk_begin + 4 * (s + 3), wave, lane, dof, voff, pc);
    }
#ifdef MSA_PHASE_TRACE
    // per item and wave (8 slots per item, whatever W): steps, the six phase
    // sums, the whole loop (clocks)
    if (a.trace && lane == 0) {
      unsigned long long* tr = a.trace + ((size_t)blockIdx.x * 8 + wave) * 8;
      tr[0] = pc.steps;
#pragma unroll
      for (int k = 0; k < 6; ++k) tr[1 + k] = pc.sum[k];
      tr[7] = clock_now() - pc.begin;
    }
#endif
  }

  // ---- epilogue ----
  write_rows<D>(a, it, ri, mrow, h, st.acc, st.m, st.l + __shfl_xor(st.l, 32, 64));
}

}  // namespace

int launch_prefill(const KernelArgs& a, int head_dim, int waves, void* stream) {
  const dim3 grid(a.n_items), block(64 * waves);
  const hipStream_t st = (hipStream_t)stream;
  if (waves != 4 && waves != 8) return (int)hipErrorInvalidValue;
  if (head_dim == 128) {
    if (waves == 8) hipLaunchKernelGGL((msa_prefill_kernel<128, 8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((msa_prefill_kernel<128, 4>), grid, block, 0, st, a);
  } else {
    if (waves == 8) hipLaunchKernelGGL((msa_prefill_kernel<64, 8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((msa_prefill_kernel<64, 4>), grid, block, 0, st, a);
  }
  return (int)hipGetLastError();
}

}  // namespace msa
