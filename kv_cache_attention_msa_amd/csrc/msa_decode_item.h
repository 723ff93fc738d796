#pragma once
// Decode work item for bf16 pools, as a device function: the body of the
// decode kernel (msa_decode.hip), also run by the chunk kernel for the decode
// tokens of a mixed batch, so that a batch of prefill chunks and decode tokens
// needs one attention launch.
//
// A decode work item: a handful of (query row, q head) pairs of one sequence
// and kv head (at most 8, e.g. one token x a GQA group) against a run of KV
// blocks.  The work is bound by HBM bandwidth: every K/V byte of the run is
// read once and used by all the rows.
//
// Work-group: 4 waves, wave w takes blocks w, w+4, w+8, ... of the item, and
// the 4 partial results are merged exactly (log-sum-exp) at the end.
// Per 16-token block, per wave:
//   * K is loaded straight into the A operand of v_mfma_f32_16x16x32_bf16
//     (lane: key lane%16; the 4 lane groups of an instruction read a 64-byte
//     run of each key row) and S^T = K Q^T gives each lane the scores of 4
//     keys for one row: the MFMA does the cross-lane reduction of the dot
//     products;
//   * V goes from the pool into a per-wave LDS buffer by LDS DMA (no
//     registers), one block ahead, its 16-byte chunks XOR-swizzled;
//   * masking (block tail, causal position) and the exponentials happen in
//     the S^T layout, against a per-row reference that moves only when needed
//     (as in the chunk kernel): in steady state a block costs no max and no
//     rescale;
//   * that layout is already the A operand of v_mfma_f32_16x16x16_bf16 (row =
//     lane % 16, keys 4 (lane / 16) .. + 3), so P stays in registers and
//     O += P V is one MFMA per 16 head_dim columns, its B operand (4 keys x one
//     column per lane) read from the V buffer with gfx950's transposing LDS
//     read;
//   * K loads for the wave's next two blocks are in flight while the current
//     one is computed.
// Slots past a block's valid count are never loaded: K reads as zero there
// and the V buffer resource covers only the valid rows, so the DMA zero-fills
// the rest (NaN in the pool never meets a 0 probability).
#include "msa_common.h"

namespace msa {
namespace dec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDecodeThreads = 256;
constexpr float kRefSumLimit = 1048576.f;  // 2^20: largest accepted partial row sum per block

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// K blocks are read exactly once per launch: non-temporal loads stream them
// past the caches instead of evicting what is still useful.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const bf16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// V of one 16-key block per wave, [wave][key][chunk]; chunk c of key row r
// sits at c ^ vsw(r).  Two of them (separate LDS variables) alternate between
// a wave's blocks, so the compiler can tell the DMA into one from the reads
// of the other.
template <int D>
struct VRing {
  uint4 v[4][kBlock][D / 8];
};

// The transposing reads take, per 16-lane group, 8 bytes of 4 consecutive key
// rows; the XOR moves each of the 4 rows to its own quarter of the banks.
template <int D>
__device__ __forceinline__ int vsw(int row) {
  return (row & 3) << (D == 128 ? 2 : 1);
}

// Per-lane byte offsets (inside a pool block) of the V chunks one DMA
// instruction brings in: instruction i fills 1 KiB of the wave's buffer, lane
// j at byte 16 j, i.e. key row i RPI + j / CPR, physical chunk j % CPR; the
// lane fetches the logical chunk that belongs there.
template <int D>
__device__ __forceinline__ uint32_t vdma_offset(int lane, int i) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int row = i * RPI + lane / CPR, pc = lane % CPR;
  return (uint32_t)(row * CPR + (pc ^ vsw<D>(row))) * 16u;
}

// Byte offset, inside a wave's V buffer, of the 8 bytes this lane addresses for
// the transposing read of head_dim columns 16 nb .. +16: lane 16 g + i
// addresses key row 4 g + i / 4, columns 16 nb + 4 (i % 4) .. + 4, so that
// after the read lane l holds V[4 (l / 16) + r][16 nb + l % 16] for r = 0..3,
// the B operand of the 16x16x16 MFMA.
template <int D>
__device__ __forceinline__ uint32_t vtr_offset(int lane, int nb) {
  const int i = lane & 15, g = lane >> 4;
  const int row = 4 * g + (i >> 2);
  const int c4 = 16 * nb + 4 * (i & 3);          // first column
  const int lc = c4 >> 3, half = (c4 >> 2) & 1;  // logical 16-byte chunk, which 8 bytes of it
  return (uint32_t)(row * (2 * D) + ((lc ^ vsw<D>(row)) << 4) + 8 * half);
}

struct BlockMeta {
  int phys, pos0, valid;
};

// Block i of the item (valid = 0 past its end: nothing is loaded for it).
__device__ __forceinline__ BlockMeta block_meta(const KernelArgs& a, const WorkItem& it, int i) {
  if (i >= it.blk_end - it.blk_begin) return BlockMeta{0, 0, 0};
  const BlockEntry e = a.blocks[it.blk_begin + i];
  return BlockMeta{entry_block(e), e.pos0, entry_valid(e)};
}

template <int D>
__device__ __forceinline__ void load_k(const KernelArgs& a, int kv_head, const BlockMeta& b, uint4 (&k)[D / 32],
                                       int lane) {
  const bf16_t* __restrict__ K = (const bf16_t*)a.k;
  const int64_t base = ((int64_t)b.phys * a.num_kv_heads + kv_head) * (kBlock * D);
  const int key = lane & 15, grp = lane >> 4;
  const bool kok = key < b.valid;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)   // chunk 4 ks + grp of the key row: one 64-byte run per key per instruction
    k[ks] = kok ? load_stream(K + base + key * D + (4 * ks + grp) * 8) : make_uint4(0, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void dma_v(const KernelArgs& a, int kv_head, const BlockMeta& b, VRing<D>& vr, int wave,
                                      int lane) {
  constexpr int RPI = 64 / (D / 8);
  const char* p = (const char*)a.v + ((int64_t)b.phys * a.num_kv_heads + kv_head) * (kBlock * D * 2);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, b.valid * D * 2, 0x00020000);
  if (a.stream_kv) {   // non-temporal: a launch whose K/V does not fit the caches (the last argument: nt)
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)&vr.v[wave][i * RPI][0], 16,
                                               (int)vdma_offset<D>(lane, i), 0, 0, 2);
  } else {
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)&vr.v[wave][i * RPI][0], 16,
                                               (int)vdma_offset<D>(lane, i), 0, 0, 0);
  }
}

// One block b: V of the next block bn goes into the other buffer vn, K of the
// block after it (bnn) into b's K registers once b's QK product has read
// them; then b's softmax against the row reference and O += P V from vr.
template <int D>
__device__ __forceinline__ void decode_block(const KernelArgs& a, const WorkItem& it, const BlockMeta& b,
                                             const BlockMeta& bn, const BlockMeta& bnn, uint4 (&k)[D / 32],
                                             const bf16x8 (&qop)[D / 32], const VRing<D>& vr, VRing<D>& vn, int wave,
                                             int lane, bool row_ok, int qpos, float& mref, float& lsum,
                                             f32x4 (&acc)[D / 16]) {
  const int grp = lane >> 4;
  const float c2 = a.scale_log2;
  dma_v<D>(a, it.kv_head, bn, vn, wave, lane);
  // ---- scores: S^T (keys x rows); lane holds keys 4 grp + r of row lane % 16 ----
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[ks]), qop[ks], s, 0, 0, 0);
  load_k<D>(a, it.kv_head, bnn, k, lane);
  // key 4 grp + r is visible iff it is below lim (positions run with the slot)
  const int lim = !row_ok ? 0 : (a.causal ? min(b.valid, qpos - b.pos0 + 1) : b.valid);
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = 4 * grp + r < lim ? s[r] * c2 : kNegInf;
  // ---- softmax against the row reference; move it only when needed ----
  float p[4];
  float mu = mref == kNegInf ? 0.f : mref;
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(x[r] - mu);
  float bs = (p[0] + p[1]) + (p[2] + p[3]);
  if (__builtin_amdgcn_ballot_w64(lim > 0 && (mref == kNegInf || !(bs <= kRefSumLimit)))) {
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool grow = mx != kNegInf && (mref == kNegInf || mx > mref + 8.f);
    const float alpha = grow ? __builtin_amdgcn_exp2f(mref - mx) : 1.f;  // mref = -inf: 0
    mref = grow ? mx : mref;
    lsum *= alpha;
    // O holds rows 4 grp + i of every column: their factors live in lanes 4 grp + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float al = __shfl(alpha, 4 * grp + i, 64);
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) acc[nb][i] *= al;
    }
    mu = mref == kNegInf ? 0.f : mref;
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(x[r] - mu);
    bs = (p[0] + p[1]) + (p[2] + p[3]);
  }
  lsum += bs;
  // ---- O += P V: A = P (row lane % 16, keys 4 grp + r), B = V^T by transposing reads ----
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 p01 = {p[0], p[1]}, p23 = {p[2], p[3]};
  const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p01, bf16x2));
  const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p23, bf16x2));
  const s16x4 pa = __builtin_bit_cast(s16x4, make_uint2(w0, w1));
  const char* vb = (const char*)&vr.v[wave][0][0];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + vtr_offset<D>(lane, nb)));
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vt, acc[nb], 0, 0, 0);
  }
}

// One decode work item on a work-group of 4 waves (256 threads).  vr0 and vr1
// are the two V buffers; after the blocks, vr0 holds the waves' partial
// outputs and vr1 their row references and sums for the merge.
template <int D, int NM>
__device__ __forceinline__ void decode_item(const KernelArgs& a, const WorkItem& it, VRing<D>& vr0, VRing<D>& vr1) {
  static_assert(sizeof(float) * 4 * NM * D <= sizeof(VRing<D>), "partial outputs must fit one V buffer");
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int col = lane & 15;     // S^T column = row of the tile
  const int grp = lane >> 4;     // S^T keys 4 grp .. 4 grp + 3
  const int g = a.group;
  const int n_mrows = it.n_q * g;
  const bool row_ok = col < n_mrows;
  const int token = it.q_row0 + (row_ok ? col / g : 0);
  const int head = it.kv_head * g + (row_ok ? col % g : 0);
  const int qpos = row_ok ? a.q_pos[token] : INT_MIN;

  bf16x8 qop[D / 32];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + ((int64_t)token * a.num_q_heads + head) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qop[ks] = as_bf16x8(row_ok ? *(const uint4*)(qrow + (4 * ks + grp) * 8) : make_uint4(0, 0, 0, 0));
  }
  f32x4 acc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) acc[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mref = kNegInf, lsum = 0.f;

  // The wave's blocks are j = 0, 1, ... (item block wave + 4 j).  While block
  // j is computed, V of block j + 1 is on its way into the other LDS buffer
  // and K of block j + 1 is in registers; K of block j + 2 is requested as
  // soon as block j's QK product has consumed its registers.
  const int nblk = it.blk_end - it.blk_begin;
  const int nj = nblk > wave ? (nblk - wave + 3) >> 2 : 0;
  if (nj > 0) {
    uint4 k0[D / 32], k1[D / 32];
    BlockMeta m0 = block_meta(a, it, wave), m1 = block_meta(a, it, wave + 4);
    load_k<D>(a, it.kv_head, m0, k0, lane);
    dma_v<D>(a, it.kv_head, m0, vr0, wave, lane);
    load_k<D>(a, it.kv_head, m1, k1, lane);
    // unrolled by two so that each block's K registers and V buffer are known
    for (int j = 0; j < nj; j += 2) {
      decode_block<D>(a, it, m0, m1, block_meta(a, it, wave + 4 * (j + 2)), k0, qop, vr0, vr1, wave, lane, row_ok,
                      qpos, mref, lsum, acc);
      if (j + 1 >= nj) break;
      m0 = block_meta(a, it, wave + 4 * (j + 2));
      decode_block<D>(a, it, m1, m0, block_meta(a, it, wave + 4 * (j + 3)), k1, qop, vr1, vr0, wave, lane, row_ok,
                      qpos, mref, lsum, acc);
      m1 = block_meta(a, it, wave + 4 * (j + 3));
    }
  }

  // ---- merge the 4 waves and write ----
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  __syncthreads();   // every wave is done with its V buffers: vr0 and vr1 become merge buffers
  float(&so)[4][NM][D] = *reinterpret_cast<float(*)[4][NM][D]>(&vr0);
  float* sm = reinterpret_cast<float*>(&vr1);   // [0, 4 NM): references, [4 NM, 8 NM): sums
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * grp + i;
      if (row < NM) so[wave][row][16 * nb + col] = acc[nb][i];
    }
  if (grp == 0 && col < NM) {
    sm[wave * NM + col] = mref;
    sm[4 * NM + wave * NM + col] = lsum;
  }
  __syncthreads();
  for (int idx = t; idx < NM * D; idx += kDecodeThreads) {
    const int mm = idx / D, d = idx % D;
    if (mm >= n_mrows) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w * NM + mm]);
    float num = 0.f, den = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = sm[w * NM + mm];
        const float wt = mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        num += wt * so[w][mm][d];
        den += wt * sm[4 * NM + w * NM + mm];
      }
    }
    const bool any = den > 0.f;
    const float o = any ? num / den : 0.f;
    const int tok = it.q_row0 + mm / g;
    const int hd = it.kv_head * g + mm % g;
    const float lse_v = any ? (M + log2f(den)) * kLn2 : kNegInf;
    if (it.part_row < 0) {
      ((bf16_t*)a.out)[((int64_t)tok * a.num_q_heads + hd) * D + d] = f32_to_bf16(o);
      if (d == 0 && a.lse) a.lse[(int64_t)tok * a.num_q_heads + hd] = lse_v;
    } else {
      a.part_o[(int64_t)(it.part_row + mm) * D + d] = o;
      if (d == 0) a.part_lse[it.part_row + mm] = lse_v;
    }
  }
}

// For the waves of a larger work-group that take no part in its decode item:
// the work-group barriers decode_item executes (exactly two, both after its
// block loop), so that every wave of the work-group reaches each of them.
__device__ __forceinline__ void decode_item_idle() {
  __syncthreads();
  __syncthreads();
}

}  // namespace dec
}  // namespace msa
