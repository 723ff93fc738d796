// Chunk (prefill) kernel for bf16 pools: exact softmax attention of a tile of
// 128 (query row, q head) pairs against a run of KV blocks, with both matrix
// products on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Work-group: 4 waves; wave w owns tile rows 32w..32w+31; two work-groups
// share a CU.  A tile row is a (query row, head of the kv head's GQA group)
// pair, so the K/V tile staged in LDS serves every q head of the group.
//
// Per step of 64 keys (4 pool blocks of the position-ordered block list, which
// may span segment boundaries):
//   * the next step's K and V are fetched from HBM into registers (16-byte
//     buffer loads, one buffer resource per pool block, whose 4 KiB per kv
//     head are contiguous) while this step computes, then written to the
//     other LDS buffer: K row-major with 16-byte chunks XOR-swizzled, V
//     transposed (head_dim rows of 64 keys) so that the PV operand is a
//     16-byte LDS read;
//   * S^T = K Q^T (K from LDS, Q^T resident in registers), so each lane holds
//     one tile row's scores for 16 keys;
//   * keys outside a block's valid slots, past the item's blocks, or (causal)
//     at a position after the row's query position get score -inf by select;
//     steps that are entirely visible to every row skip the mask;
//   * online softmax in the exp2 domain (scale * log2 e folded into one FMA)
//     against a per-row reference that moves only when needed;
//   * P is rounded to bf16 in place of the S accumulator registers and used as
//     the B operand of O^T += V^T P^T.
// Slots that hold no key are zero-filled in LDS, so the 0-probabilities never
// meet pool contents (NaN * 0 would poison the row).
#include "msa_common.h"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kStepKeys = 64;   // keys per step = 4 blocks
constexpr float kRefSumLimit = 1048576.f;  // 2^20: largest accepted partial row sum per step

// LDS tiles.  Operand reads touch 32 consecutive rows at one chunk index; the
// XOR swizzles below were chosen by measurement on gfx950 so that those reads
// run at the rate of a contiguous ds_read_b128 (about 4.4 clocks per wave
// instruction per CU) and the staging writes at the rate of contiguous writes.
template <int D>
struct PrefillSmem {
  uint4 k[2][kStepKeys][D / 8];   // [buf][key][chunk]: K rows (head_dim), swizzled
  uint4 vt[2][D][kStepKeys / 8];  // [buf][d][chunk]: V transposed (64 keys), swizzled
};

// K rows are 256 bytes (D=128: one row covers all banks) or 128 bytes (D=64:
// rows of one parity share a bank half).
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}
// Vt rows are 128 bytes.  With (d >> 1) ^ (d >> 4) both the operand reads and
// the transposed staging writes (rows 8 apart) are conflict-free; the
// (d >> 1) ^ (d >> 3) variant halves the operand-read rate.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

// Position of local key k (0..63) inside a transposed V row: bits 2 and 3 of
// k are swapped so that the 8 keys one lane feeds to the PV MFMA are adjacent.
__device__ __forceinline__ int vt_key_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

template <int D>
__device__ __forceinline__ bf16x8 ld_k(const PrefillSmem<D>& sm, int buf, int row, int c) {
  return as_bf16x8(sm.k[buf][row][c ^ k_swz<D>(row)]);
}
template <int D>
__device__ __forceinline__ bf16x8 ld_vt(const PrefillSmem<D>& sm, int buf, int d, int c) {
  return as_bf16x8(sm.vt[buf][d][c ^ vt_swz(d)]);
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
// pool block ids, so loads from them stay in bounds).
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

template <int D>
struct StepRegs {
  uint4 k[D / 32];   // D=128: 4 chunks, D=64: 2 chunks
  uint4 v[D / 32];   // keys-per-thread of one 16-byte d chunk
};

// Global -> registers for one step.  Every load is in bounds (block ids of
// the step are pool ids, slots 0..15); slots that hold no key are dealt with
// later (K: masked scores, V: zeroed when staged).  K and V are fetched at
// different points of a step so that their staging registers are not live
// at the same time.
// One pool block of one kv head as a buffer resource (scalar registers):
// loads take a 32-bit lane offset, and offsets past the block read zero.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* pool, int kv_head, int num_kv_heads, int phys) {
  const char* p = (const char*)pool + ((int64_t)phys * num_kv_heads + kv_head) * (kBlock * D * 2);
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, kBlock * D * 2, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int D>
__device__ __forceinline__ void fetch_k(const KernelArgs& a, int kv_head, const StepMeta& m, StepRegs<D>& r, int t) {
  constexpr int CPR = D / 8;  // 16-byte chunks per key row
  // D = 128: chunk i*256+t is block i, row t/16, chunk t%16.
  // D = 64:  chunk i*256+t is block 2i + t/128, row (t/8)%16, chunk t%8.
  const uint32_t off = (D == 128) ? (uint32_t)t * 16u : (uint32_t)(((t >> 3) & 15) * D + (t % CPR) * 8) * 2u;
  const int half = __builtin_amdgcn_readfirstlane(t >> 7);
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int b = (D == 128) ? i : 2 * i + half;
    r.k[i] = buf_load16(block_rsrc<D>(a.k, kv_head, a.num_kv_heads, m.phys(b)), off);
  }
}
template <int D>
__device__ __forceinline__ void fetch_v(const KernelArgs& a, int kv_head, const StepMeta& m, StepRegs<D>& r, int t) {
  constexpr int CPR = D / 8;
  constexpr int KPT = D / 32;            // keys per thread for V
  const int c = t % CPR, kg = t / CPR;
  // a wave's keys lie in one block: D = 128, block = wave; D = 64, wave / 2
  const int b = __builtin_amdgcn_readfirstlane((kg * KPT) >> 4);
  const uint32_t off = (uint32_t)(((kg * KPT) & 15) * D + c * 8) * 2u;
  const __amdgpu_buffer_rsrc_t rs = block_rsrc<D>(a.v, kv_head, a.num_kv_heads, m.phys(b));
#pragma unroll
  for (int e = 0; e < KPT; ++e) r.v[e] = buf_load16(rs, off + e * D * 2);
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// Registers -> LDS buffer: K row-major swizzled; V transposed, with V rows of
// slots without a key written as zero on steps that are not full.
template <int D>
__device__ __forceinline__ void stage_k(PrefillSmem<D>& sm, int buf, const StepRegs<D>& r, int t) {
  // Chunk i*256+t goes to row i*(4096/(2D)) + t/CPR; the swizzle of that row
  // does not depend on i, so the rows of one lane are 4 KiB apart.
  constexpr int CPR = D / 8;
  const int row = t / CPR, c = t % CPR;
  char* dst = (char*)&sm.k[buf][row][c ^ k_swz<D>(row)];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) *(uint4*)(dst + i * 4096) = r.k[i];
}
template <int D>
__device__ __forceinline__ void stage_v(PrefillSmem<D>& sm, int buf, StepRegs<D>& r, const StepMeta& m, int t) {
  constexpr int CPR = D / 8;
  constexpr int KPT = D / 32;
  const int c = t % CPR, kg = t / CPR;
  if (!m.full) {
    // a wave's keys lie in one block
    const int b = __builtin_amdgcn_readfirstlane((kg * KPT) >> 4);
    const int valid = b < m.nb ? m.valid(b) : 0;
    const int slot0 = (kg * KPT) & 15;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const bool dead = slot0 + e >= valid;
      r.v[e].x = dead ? 0u : r.v[e].x;
      r.v[e].y = dead ? 0u : r.v[e].y;
      r.v[e].z = dead ? 0u : r.v[e].z;
      r.v[e].w = dead ? 0u : r.v[e].w;
    }
  }
  const int kpos = vt_key_pos(kg * KPT);
  const int chunk = kpos >> 3;
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int d = c * 8 + dd;
    const int w = dd >> 1;
    // bytes {0,1} (even dd) or {2,3} (odd dd) of word w of each key, low key first
    const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
    char* dst = (char*)&sm.vt[buf][d][chunk ^ vt_swz(d)] + (kpos & 7) * 2;
    if constexpr (KPT == 4) {
      *(uint2*)dst = make_uint2(__builtin_amdgcn_perm(word_of(r.v[1], w), word_of(r.v[0], w), sel),
                                __builtin_amdgcn_perm(word_of(r.v[3], w), word_of(r.v[2], w), sel));
    } else {
      *(uint32_t*)dst = __builtin_amdgcn_perm(word_of(r.v[1], w), word_of(r.v[0], w), sel);
    }
  }
}

// Scores of one 32-row half for a step: s{kb} register r holds key
// 32kb + 8(r/4) + 4h + r%4 (block 2kb + r/8, slot 8((r/4)&1) + 4h + r%4).
__device__ __forceinline__ void mask_half(f32x16& s0, f32x16& s1, const StepMeta& m, int h, int qpos, bool causal) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int slot = 8 * ((r >> 2) & 1) + 4 * h + (r & 3);
    const int b0 = r >> 3, b1 = 2 + (r >> 3);
    const bool ok0 = slot < m.valid(b0) && (!causal || m.pos0(b0) + slot <= qpos);
    const bool ok1 = slot < m.valid(b1) && (!causal || m.pos0(b1) + slot <= qpos);
    s0[r] = ok0 ? s0[r] : kNegInf;
    s1[r] = ok1 ? s1[r] : kNegInf;
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

template <int D>
__global__ __launch_bounds__(kThreads, 2) void msa_prefill_kernel(KernelArgs a) {
  __shared__ PrefillSmem<D> sm;
  const WorkItem it = a.items[blockIdx.x];
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int h = lane >> 5;        // lane half: which 8 of each 16 reduction indices
  const int col = lane & 31;      // tile row within the wave
  const int mrow = wave * 32 + col;
  const RowInfo ri = row_info(a, it, mrow);

  // Q^T operand: lane holds q[row][16ks + 8h .. +8) for every ks.
  bf16x8 qop[D / 16];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + ((int64_t)ri.token * a.num_q_heads + ri.head) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qop[ks] = as_bf16x8(ri.ok ? *(const uint4*)(qrow + ks * 16 + h * 8) : make_uint4(0, 0, 0, 0));
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){0};
  float m = kNegInf, l = 0.f;
  const float c2 = a.scale_log2;

  const int nblk = it.blk_end - it.blk_begin;
  const int nsteps = (nblk + 3) >> 2;
  if (nsteps > 0) {
    StepMeta cur, nxt;
    StepRegs<D> regs;
    load_meta(a, it.blk_begin, it.blk_end, it.q_min, cur);
    fetch_k<D>(a, it.kv_head, cur, regs, t);
    fetch_v<D>(a, it.kv_head, cur, regs, t);
    stage_k<D>(sm, 0, regs, t);
    stage_v<D>(sm, 0, regs, cur, t);
    load_meta(a, it.blk_begin + 4, it.blk_end, it.q_min, nxt);
    __syncthreads();

    for (int s = 0; s < nsteps; ++s) {
      const int buf = s & 1;
      // Next step's K (a step past the item's end reads in-bounds pool blocks
      // and is never used).
      fetch_k<D>(a, it.kv_head, nxt, regs, t);

      // ---- S^T = K Q^T for 64 keys ----
      f32x16 s0 = (f32x16){0}, s1 = (f32x16){0};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 k0 = ld_k<D>(sm, buf, col, 2 * ks + h);
        const bf16x8 k1 = ld_k<D>(sm, buf, 32 + col, 2 * ks + h);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qop[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qop[ks], s1, 0, 0, 0);
      }
      stage_k<D>(sm, buf ^ 1, regs, t);
      fetch_v<D>(a, it.kv_head, nxt, regs, t);

      if (!cur.full) mask_half(s0, s1, cur, h, ri.qpos, a.causal);

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
      float rs = exp_half(s0, s1, c2, m == kNegInf ? 0.f : m, pw);
      if (__builtin_amdgcn_ballot_w64(m == kNegInf || !(rs <= kRefSumLimit))) {
        const float mx = row_max(s0, s1) * c2;
        const bool grow = mx != kNegInf && (m == kNegInf || mx > m + 8.f);
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mx) : 1.f;  // m = -inf: 0
        m = grow ? mx : m;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
        rs = exp_half(s0, s1, c2, m == kNegInf ? 0.f : m, pw);
      }
      l += rs;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int w0 = (ks >> 1) * 8 + (ks & 1) * 4;
        const bf16x8 pop = as_bf16x8(make_uint4(pw[w0], pw[w0 + 1], pw[w0 + 2], pw[w0 + 3]));
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 v = ld_vt<D>(sm, buf, db * 32 + col, 2 * ks + h);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pop, acc[db], 0, 0, 0);
        }
      }

      stage_v<D>(sm, buf ^ 1, regs, nxt, t);
      cur = nxt;
      load_meta(a, it.blk_begin + 4 * (s + 2), it.blk_end, it.q_min, nxt);
      __syncthreads();
    }
  }

  // ---- epilogue ----
  write_rows<D>(a, it, ri, mrow, h, acc, m, l + __shfl_xor(l, 32, 64));
}

}  // namespace

int launch_prefill(const KernelArgs& a, int head_dim, void* stream) {
  dim3 grid(a.n_items), block(kThreads);
  if (head_dim == 128)
    hipLaunchKernelGGL(msa_prefill_kernel<128>, grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(msa_prefill_kernel<64>, grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace msa
