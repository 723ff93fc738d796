// Row-at-a-time MSA kernel for fp32 pools.
//
// One wave owns one (query row, q head) pair and walks the work item's KV
// blocks in position order, a whole block (16 keys) at a time: lanes split
// head_dim, the 16 key rows of a block are loaded together (one memory
// latency per block, not per key), each key's score is a wave-wide sum, and a
// running max / running sum / running output over blocks give exact softmax
// (Eq. 1) in one pass.  Slots past a block's valid count, and (causal) keys
// after the row's position, get probability 0 by select; a causal row stops
// at the first block that starts after its position (positions increase along
// the block list).
#include "msa_common.h"

namespace msa {

constexpr int kFp32Threads = kFp32MRows * 64;   // one wave per tile row

template <typename T, int D>
__device__ __forceinline__ void rowwise_row(const KernelArgs& a, const WorkItem& it, const T* __restrict__ K,
                                            const T* __restrict__ V, int mr, int lane);

template <typename T, int D>
__global__ __launch_bounds__(kFp32Threads) void msa_rowwise_kernel(KernelArgs a) {
  const WorkItem it = a.items[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int g = a.group;
  const T* __restrict__ K = (const T*)a.k;
  const T* __restrict__ V = (const T*)a.v;
  // a tile has more rows than waves only when one token's GQA group does
  for (int mr = threadIdx.x >> 6; mr < it.n_q * g; mr += kFp32MRows)
    rowwise_row<T, D>(a, it, K, V, mr, lane);
}

template <typename T, int D>
__device__ __forceinline__ void rowwise_row(const KernelArgs& a, const WorkItem& it, const T* __restrict__ K,
                                            const T* __restrict__ V, int mr, int lane) {
  constexpr int E = D / 64;  // elements of head_dim per lane
  const int g = a.group;
  const int row = it.q_row0 + mr / g;
  const int head = it.kv_head * g + mr % g;
  const int qp = a.q_pos[row];
  const T* qrow = (const T*)a.q + ((int64_t)row * a.num_q_heads + head) * D;
  float qv[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = to_f32<T>(qrow[lane * E + e]);
    acc[e] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  for (int b = it.blk_begin; b < it.blk_end; ++b) {
    const BlockEntry be = a.blocks[b];
    int nvis = entry_valid(be);
    if (a.causal) nvis = min(nvis, qp - be.pos0 + 1);
    if (nvis <= 0) break;   // this block, and every later one, starts after the row
    const int64_t base = ((int64_t)entry_block(be) * a.num_kv_heads + it.kv_head) * (int64_t)(kBlock * D);
    float x[kBlock];
#pragma unroll
    for (int s = 0; s < kBlock; ++s) {
      const T* kr = K + base + s * D;   // inside the block: every slot is readable
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) dot += qv[e] * to_f32<T>(kr[lane * E + e]);
      x[s] = dot;
    }
    float mx = kNegInf;
#pragma unroll
    for (int s = 0; s < kBlock; ++s) {
      x[s] = s < nvis ? wave_sum(x[s]) * a.scale_log2 : kNegInf;
      mx = fmaxf(mx, x[s]);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
#pragma unroll
    for (int s = 0; s < kBlock; ++s) {
      const float pr = s < nvis ? exp2f(x[s] - mn) : 0.f;
      const T* vr = V + base + s * D;
      l += pr;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float v = to_f32<T>(vr[lane * E + e]);
        acc[e] += s < nvis ? pr * v : 0.f;   // select: a slot without a key may hold NaN
      }
    }
    m = mn;
  }
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const float lse_v = any ? (m + log2f(l)) * kLn2 : kNegInf;
  if (it.part_row < 0) {
    T* orow = (T*)a.out + ((int64_t)row * a.num_q_heads + head) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[lane * E + e] = from_f32<T>(acc[e] * inv);
    if (a.lse && lane == 0) a.lse[(int64_t)row * a.num_q_heads + head] = lse_v;
  } else {
    float* prow = a.part_o + (int64_t)(it.part_row + mr) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) prow[lane * E + e] = acc[e] * inv;
    if (lane == 0) a.part_lse[it.part_row + mr] = lse_v;
  }
}

template <typename T>
static int launch_rowwise(const KernelArgs& a, int head_dim, void* stream) {
  dim3 grid(a.n_items), block(kFp32Threads);
  if (head_dim == 128)
    hipLaunchKernelGGL((msa_rowwise_kernel<T, 128>), grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((msa_rowwise_kernel<T, 64>), grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_fp32(const KernelArgs& a, int head_dim, void* stream) {
  return launch_rowwise<float>(a, head_dim, stream);
}

}  // namespace msa
