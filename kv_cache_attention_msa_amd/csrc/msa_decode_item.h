#pragma once
// Decode work item for bf16 pools, as a device function: the body of the
// decode kernel (msa_decode.hip), also run by the chunk kernel for the decode
// tokens of a mixed batch, so that a batch of prefill chunks and decode tokens
// needs one attention launch.
//
// A decode work item: a handful of (query row, q head) pairs of one
// sequence and kv head (at most 8, e.g. one token x a GQA group) against a
// run of KV blocks.  The work is bound by HBM bandwidth: every K/V byte of
// the run is read once and used by all the rows.
//
// Work-group: 4 waves, wave w takes blocks w, w+4, w+8, ... of the item, and
// the 4 partial results are merged exactly (log-sum-exp) at the end.
// Per 16-token block, per wave:
//   * K is loaded straight into the A operand of v_mfma_f32_16x16x32_bf16
//     (lane: key lane%16; the 4 lane groups of an instruction read a 64-byte
//     run of each key row) and S^T = K Q^T gives each
//     lane the scores of 4 keys for one row: the MFMA does the cross-lane
//     reduction of the dot products;
//   * masking (block tail, causal position), running max and exp2 happen in
//     that layout; the probabilities and the rescale factor go through a small
//     per-wave LDS slot;
//   * V is read with fully coalesced 16-byte loads (4 keys x 256 bytes per
//     instruction) and accumulated as fp32 FMAs: each lane owns 8 head_dim
//     columns of every row;
//   * loads for the wave's next two blocks are in flight while the current one
//     is computed.
// Slots past a block's valid count are never loaded (V reads as zero there).
#include "msa_common.h"

namespace msa {
namespace dec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecodeThreads = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// K/V blocks are read exactly once per launch: non-temporal loads stream them
// past the caches instead of evicting what is still useful (measured on the
// 64-sequence decode: 238 -> 216 us).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const bf16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

struct BlockMeta {
  int phys, pos0, valid;
};

__device__ __forceinline__ BlockMeta block_meta(const KernelArgs& a, int idx) {
  const BlockEntry e = a.blocks[idx];
  return BlockMeta{entry_block(e), e.pos0, entry_valid(e)};
}

template <int D>
struct DecodeRegs {
  uint4 k[D / 32];   // A operand chunks, one per MFMA k-step
  uint4 v[D / 32];   // 16-byte V chunks (keys KPL*j + lane / CPR)
};

template <int D>
__device__ __forceinline__ void fetch_block(const KernelArgs& a, int kv_head, const BlockMeta& b,
                                            DecodeRegs<D>& r, int lane) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 32;
  constexpr int KPL = 64 / CPR;
  const bf16_t* __restrict__ K = (const bf16_t*)a.k;
  const bf16_t* __restrict__ V = (const bf16_t*)a.v;
  const int64_t base = ((int64_t)b.phys * a.num_kv_heads + kv_head) * (kBlock * D);
  const int key = lane & 15, grp = lane >> 4;
  const bool kok = key < b.valid;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    // this lane's 16-byte chunk for k-step ks: the 4 lane groups read one
    // contiguous 64-byte run of each key row per instruction
    const int c = 4 * ks + grp;
    r.k[ks] = kok ? load_stream(K + base + key * D + c * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const int vk = KPL * j + lane / CPR;
    r.v[j] = vk < b.valid ? load_stream(V + base + vk * D + (lane % CPR) * 8) : make_uint4(0, 0, 0, 0);
  }
}

// Shared memory of one decode work-group (4 waves).
template <int D, int NM>
struct DecodeShared {
  float sp[4][17][NM];        // per wave: p[key][row]; row 16 holds the rescale factors
  float sm_m[4][NM], sm_l[4][NM];
  float so[4][NM][D];
};

// One decode work item on a work-group of 4 waves (256 threads).
template <int D, int NM>
__device__ __forceinline__ void decode_item(const KernelArgs& a, const WorkItem& it, DecodeShared<D, NM>& sh) {
  constexpr int CPR = D / 8;     // 16-byte chunks per key row
  constexpr int KS = D / 32;     // MFMA k-steps
  constexpr int KPL = 64 / CPR;  // keys per V load instruction
  constexpr int VL = 16 / KPL;   // V load instructions per block (== KS)
  static_assert(VL == KS, "layout");
  auto& sp = sh.sp;
  auto& sm_m = sh.sm_m;
  auto& sm_l = sh.sm_l;
  auto& so = sh.so;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int col = lane & 15;     // S^T column = row of the tile
  const int grp = lane >> 4;     // S^T keys 4*grp .. 4*grp+3
  const int g = a.group;
  const int n_mrows = it.n_q * g;
  const bool row_ok = col < n_mrows;
  const int token = it.q_row0 + (row_ok ? col / g : 0);
  const int head = it.kv_head * g + (row_ok ? col % g : 0);
  const int qpos = row_ok ? a.q_pos[token] : INT_MIN;
  const float c2 = a.scale_log2;

  bf16x8 qop[KS];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + ((int64_t)token * a.num_q_heads + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = as_bf16x8(row_ok ? *(const uint4*)(qrow + (4 * ks + grp) * 8) : make_uint4(0, 0, 0, 0));
  }

  float acc[NM][8];
#pragma unroll
  for (int mm = 0; mm < NM; ++mm)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[mm][e] = 0.f;
  float m = kNegInf, lsum = 0.f;

  const int nblk = it.blk_end - it.blk_begin;
  int i = wave;
  if (i < nblk) {
    // Register ring of the wave's blocks i, i+4, i+8: two blocks are in flight
    // while one is computed.  Indices past the item's end are clamped to its
    // last block (in-bounds loads whose data is never used).
    DecodeRegs<D> cur, nxt, nxt2;
    BlockMeta mc = block_meta(a, it.blk_begin + i);
    BlockMeta mn = block_meta(a, it.blk_begin + min(i + 4, nblk - 1));
    BlockMeta mn2 = block_meta(a, it.blk_begin + min(i + 8, nblk - 1));
    fetch_block<D>(a, it.kv_head, mc, cur, lane);
    fetch_block<D>(a, it.kv_head, mn, nxt, lane);
    for (; i < nblk; i += 4) {
      fetch_block<D>(a, it.kv_head, mn2, nxt2, lane);
      const BlockMeta mn3 = block_meta(a, it.blk_begin + min(i + 12, nblk - 1));

      // ---- scores: S^T (keys x rows), lane holds keys 4*grp+r of row col ----
      f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.k[ks]), qop[ks], s, 0, 0, 0);
      const bool full = mc.valid == 16 && (!a.causal || mc.pos0 + 15 <= it.q_min);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 4 * grp + r;
        const bool ok = full ? row_ok : (row_ok && slot < mc.valid && (!a.causal || mc.pos0 + slot <= qpos));
        x[r] = ok ? s[r] * c2 : kNegInf;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(x[r] - m_use);
      lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m = m_new;
      if (col < NM) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sp[wave][4 * grp + r][col] = p[r];
        if (grp == 0) sp[wave][16][col] = alpha;
      }
      wave_sync_lds();

      // ---- O += P V (fp32 FMAs; lane owns 8 columns of every row) ----
#pragma unroll
      for (int mm = 0; mm < NM; ++mm) {
        const float al = sp[wave][16][mm];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[mm][e] *= al;
      }
#pragma unroll
      for (int j = 0; j < VL; ++j) {
        const int key = KPL * j + lane / CPR;
        const uint4 u = cur.v[j];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[2 * e] = __uint_as_float(w[e] << 16);
          vf[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
#pragma unroll
        for (int mm = 0; mm < NM; ++mm) {
          const float pm = sp[wave][key][mm];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[mm][e] = fmaf(pm, vf[e], acc[mm][e]);
        }
      }
      wave_sync_lds();

      cur = nxt;
      nxt = nxt2;
      mc = mn;
      mn = mn2;
      mn2 = mn3;
    }
  }

  // ---- reduce within the wave: lanes with equal (lane % CPR) own the same columns ----
#pragma unroll
  for (int mm = 0; mm < NM; ++mm)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[mm][e];
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[mm][e] = v;
    }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (lane < CPR) {
#pragma unroll
    for (int mm = 0; mm < NM; ++mm)
#pragma unroll
      for (int e = 0; e < 8; ++e) so[wave][mm][lane * 8 + e] = acc[mm][e];
  }
  if (grp == 0 && col < NM) {
    sm_m[wave][col] = m;
    sm_l[wave][col] = lsum;
  }
  __syncthreads();

  // ---- merge the 4 waves and write ----
  for (int idx = t; idx < NM * D; idx += kDecodeThreads) {
    const int mm = idx / D, d = idx % D;
    if (mm >= n_mrows) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][mm]);
    float num = 0.f, den = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float wt = __builtin_amdgcn_exp2f(sm_m[w][mm] - M);
        num += wt * so[w][mm][d];
        den += wt * sm_l[w][mm];
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


}  // namespace dec
}  // namespace msa
