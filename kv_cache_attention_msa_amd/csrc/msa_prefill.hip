// Chunk (prefill) kernel for bf16 pools: exact softmax attention of a tile of
// 128 (query row, q head) pairs against a run of KV blocks, with both matrix
// products on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Work-group: 4 waves; wave w owns tile rows 32w..32w+31.  A tile row is a
// (query row, head of the kv head's GQA group) pair, so the K/V tile staged in
// LDS serves every q head of the group.
//
// Per step of 64 keys (4 pool blocks of the position-ordered block list, which
// may span segment boundaries):
//   * the next step's K and V are fetched from HBM into registers (16-byte
//     loads; one block's 4 KiB are contiguous) while this step computes, then
//     written to the other LDS buffer: K row-major with 16-byte chunks XOR-
//     swizzled, V transposed (head_dim rows of 64 keys) so that the PV operand
//     is a 16-byte LDS read;
//   * S^T = K Q^T (K from LDS, Q^T resident in registers), so each lane holds
//     one tile row's scores for 16 keys;
//   * keys outside a block's valid slots, past the item's blocks, or (causal)
//     at a position after the row's query position get score -inf by select;
//     steps that are entirely visible to every row skip the mask;
//   * online softmax in the exp2 domain (scale * log2 e folded into one FMA);
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

template <int D>
struct PrefillSmem {
  uint4 k[2][kStepKeys * D / 8];   // [key][D], 16-byte chunks swizzled
  uint4 vt[2][D * kStepKeys / 8];  // [d][64 keys], keys permuted, chunks swizzled
};

// XOR swizzle of 16-byte chunks for rows of 8 chunks (128 bytes): any 8
// consecutive rows, and any 16 consecutive rows of one parity, map a chunk
// index to distinct chunk positions.
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

template <int D>
__device__ __forceinline__ int k_chunk(int row, int c) {
  if constexpr (D == 128) return row * 16 + (c ^ (row & 15));
  else return row * 8 + (c ^ swz8(row));
}
__device__ __forceinline__ int vt_chunk(int d, int c) { return d * 8 + (c ^ swz8(d)); }

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

// Descriptors of one step's (up to) 4 blocks.  Plain scalar fields rather
// than arrays, so that no private array is ever indexed at run time.
struct StepMeta {
  int nb;                          // blocks in this step (1..4)
  int ph0, ph1, ph2, ph3;          // pool block ids
  int ps0, ps1, ps2, ps3;          // positions of slot 0
  int vl0, vl1, vl2, vl3;          // valid slots (0 past the item's end)
  __device__ __forceinline__ int phys(int b) const { return b == 0 ? ph0 : b == 1 ? ph1 : b == 2 ? ph2 : ph3; }
  __device__ __forceinline__ int pos0(int b) const { return b == 0 ? ps0 : b == 1 ? ps1 : b == 2 ? ps2 : ps3; }
  __device__ __forceinline__ int valid(int b) const { return b == 0 ? vl0 : b == 1 ? vl1 : b == 2 ? vl2 : vl3; }
};

// Branch-free so that the step descriptors stay in (scalar) registers: blocks
// past the item's end re-read its last entry and get valid = 0.
__device__ __forceinline__ void load_meta(const KernelArgs& a, int blk, int blk_end, StepMeta& m) {
  m.nb = min(4, blk_end - blk);
  const BlockEntry e0 = a.blocks[blk];
  const BlockEntry e1 = a.blocks[min(blk + 1, blk_end - 1)];
  const BlockEntry e2 = a.blocks[min(blk + 2, blk_end - 1)];
  const BlockEntry e3 = a.blocks[min(blk + 3, blk_end - 1)];
  m.ph0 = a.block_table[entry_bt(e0)];
  m.ph1 = a.block_table[entry_bt(e1)];
  m.ph2 = a.block_table[entry_bt(e2)];
  m.ph3 = a.block_table[entry_bt(e3)];
  m.ps0 = e0.pos0; m.ps1 = e1.pos0; m.ps2 = e2.pos0; m.ps3 = e3.pos0;
  m.vl0 = entry_valid(e0);
  m.vl1 = m.nb > 1 ? entry_valid(e1) : 0;
  m.vl2 = m.nb > 2 ? entry_valid(e2) : 0;
  m.vl3 = m.nb > 3 ? entry_valid(e3) : 0;
}

template <int D>
struct StepRegs {
  uint4 k[D / 32];   // D=128: 4 chunks, D=64: 2 chunks
  uint4 v[D / 32];   // keys-per-thread of one 16-byte d chunk
};

// Global -> registers for one step.  Slots without a key load as zero.
template <int D>
__device__ __forceinline__ void fetch_step(const KernelArgs& a, int kv_head, const StepMeta& m,
                                           StepRegs<D>& r, int t) {
  constexpr int CPR = D / 8;  // 16-byte chunks per key row
  const bf16_t* __restrict__ K = (const bf16_t*)a.k;
  const bf16_t* __restrict__ V = (const bf16_t*)a.v;
  const int64_t head_off = (int64_t)kv_head * (kBlock * D);
  const int64_t blk_stride = (int64_t)a.num_kv_heads * (kBlock * D);
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    // D = 128: chunk i*256+t is block i, row t/16, chunk t%16.
    // D = 64:  chunk i*256+t is block 2i + t/128, row (t/8)%16, chunk t%8.
    const int b = (D == 128) ? i : 2 * i + (t >> 7);
    const int slot = (D == 128) ? (t >> 4) : ((t >> 3) & 15);
    const int c = t % CPR;
    const int phys = m.phys(b);
    const int valid = m.valid(b);
    const bool ok = b < m.nb && slot < valid;
    const uint4* src = (const uint4*)(K + phys * blk_stride + head_off + slot * D + c * 8);
    r.k[i] = ok ? *src : make_uint4(0, 0, 0, 0);
  }
  constexpr int KPT = D / 32;            // keys per thread for V
  const int c = t % CPR, kg = t / CPR;
  const int kbase = kg * KPT;
  const int b = kbase >> 4, slot0 = kbase & 15;
  const int phys = m.phys(b);
  const int valid = m.valid(b);
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const bool ok = b < m.nb && slot0 + e < valid;
    const uint4* src = (const uint4*)(V + phys * blk_stride + head_off + (slot0 + e) * D + c * 8);
    r.v[e] = ok ? *src : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// Registers -> LDS buffer (K row-major swizzled, V transposed).
template <int D>
__device__ __forceinline__ void stage_step(PrefillSmem<D>& sm, int buf, const StepRegs<D>& r, int t) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int id = i * kThreads + t;
    const int row = id / CPR, c = id % CPR;
    sm.k[buf][k_chunk<D>(row, c)] = r.k[i];
  }
  constexpr int KPT = D / 32;
  const int c = t % CPR, kg = t / CPR;
  const int kpos = vt_key_pos(kg * KPT);
  char* vbase = (char*)sm.vt[buf];
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int d = c * 8 + dd;
    const int off = vt_chunk(d, kpos >> 3) * 16 + (kpos & 7) * 2;
    const int w = dd >> 1;
    const bool hi = dd & 1;
    if constexpr (KPT == 4) {
      uint32_t x0 = word_of(r.v[0], w), x1 = word_of(r.v[1], w), x2 = word_of(r.v[2], w), x3 = word_of(r.v[3], w);
      uint2 val;
      val.x = hi ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
      val.y = hi ? ((x2 >> 16) | (x3 & 0xffff0000u)) : ((x2 & 0xffffu) | (x3 << 16));
      *(uint2*)(vbase + off) = val;
    } else {
      uint32_t x0 = word_of(r.v[0], w), x1 = word_of(r.v[1], w);
      *(uint32_t*)(vbase + off) = hi ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
    }
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
  const int g = a.group;
  const int n_mrows = it.n_q * g;
  const int mrow = wave * 32 + col;
  const bool row_ok = mrow < n_mrows;
  const int token = it.q_row0 + (row_ok ? mrow / g : 0);
  const int head = it.kv_head * g + (row_ok ? mrow % g : 0);
  const int qpos = row_ok ? a.q_pos[token] : INT_MIN;

  // Q^T operand: lane holds q[row][16ks + 8h .. +8) for every ks.
  bf16x8 qop[D / 16];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + ((int64_t)token * a.num_q_heads + head) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 u = row_ok ? *(const uint4*)(qrow + ks * 16 + h * 8) : make_uint4(0, 0, 0, 0);
      qop[ks] = as_bf16x8(u);
    }
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
    load_meta(a, it.blk_begin, it.blk_end, cur);
    fetch_step<D>(a, it.kv_head, cur, regs, t);
    stage_step<D>(sm, 0, regs, t);
    if (nsteps > 1) load_meta(a, it.blk_begin + 4, it.blk_end, nxt);
    __syncthreads();

    for (int s = 0; s < nsteps; ++s) {
      const int buf = s & 1;
      const bool more = s + 1 < nsteps;
      if (more) fetch_step<D>(a, it.kv_head, nxt, regs, t);

      // ---- S^T = K Q^T for 64 keys ----
      f32x16 s0 = (f32x16){0}, s1 = (f32x16){0};
      const uint4* kl = sm.k[buf];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 k0 = as_bf16x8(kl[k_chunk<D>(col, 2 * ks + h)]);
        const bf16x8 k1 = as_bf16x8(kl[k_chunk<D>(32 + col, 2 * ks + h)]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qop[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qop[ks], s1, 0, 0, 0);
      }

      // ---- mask: register r of s{kb} holds key 32kb + 8(r/4) + 4h + r%4,
      //      i.e. block 2kb + r/8, slot 8((r/4)&1) + 4h + r%4 ----
      const int last = cur.nb - 1;
      const bool full = cur.nb == 4 && cur.vl0 == 16 && cur.vl1 == 16 && cur.vl2 == 16 && cur.vl3 == 16 &&
                        (!a.causal || cur.ps3 + 15 <= it.q_min);
      (void)last;
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int slot = 8 * ((r >> 2) & 1) + 4 * h + (r & 3);
          const int b0 = r >> 3, b1 = 2 + (r >> 3);
          const bool ok0 = slot < cur.valid(b0) && (!a.causal || cur.pos0(b0) + slot <= qpos);
          const bool ok1 = slot < cur.valid(b1) && (!a.causal || cur.pos0(b1) + slot <= qpos);
          s0[r] = ok0 ? s0[r] : kNegInf;
          s1[r] = ok1 ? s1[r] : kNegInf;
        }
      }

      // ---- online softmax (exp2 domain) ----
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx * c2);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float rs = 0.f;
      uint32_t pw[16];  // P in bf16, two per word: word j of kb holds regs 2j, 2j+1
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s0[r + 1], c2, -m_use));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, -m_use));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(s1[r + 1], c2, -m_use));
        rs += (p0 + p1) + (p2 + p3);
        pw[r / 2] = pack_bf16x2(p0, p1);
        pw[8 + r / 2] = pack_bf16x2(p2, p3);
      }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;

      // ---- O^T += V^T P^T ----
      const uint4* vl = sm.vt[buf];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int w0 = (ks >> 1) * 8 + (ks & 1) * 4;
        const bf16x8 pop = as_bf16x8(make_uint4(pw[w0], pw[w0 + 1], pw[w0 + 2], pw[w0 + 3]));
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 v = as_bf16x8(vl[vt_chunk(db * 32 + col, 2 * ks + h)]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pop, acc[db], 0, 0, 0);
        }
      }

      if (more) {
        stage_step<D>(sm, buf ^ 1, regs, t);
        cur = nxt;
        if (s + 2 < nsteps) load_meta(a, it.blk_begin + 4 * (s + 2), it.blk_end, nxt);
      }
      __syncthreads();
    }
  }

  // ---- epilogue ----
  const float l_tot = l + __shfl_xor(l, 32, 64);
  if (!row_ok) return;
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m + log2f(l_tot)) * kLn2 : kNegInf;
  if (it.part_row < 0) {
    bf16_t* orow = (bf16_t*)a.out + ((int64_t)token * a.num_q_heads + head) * D;
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
    if (a.lse && h == 0) a.lse[(int64_t)token * a.num_q_heads + head] = lse_v;
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
