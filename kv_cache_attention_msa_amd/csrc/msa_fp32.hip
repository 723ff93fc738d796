// Row-at-a-time MSA kernel for fp32 pools.
//
// One wave owns one (query row, q head) pair at a time and walks the work
// item's KV blocks in position order: lanes split head_dim, each key's score
// is a wave-wide sum, and a running max / running sum / running output give
// exact softmax (Eq. 1) in one pass.  A block's slots beyond its valid count
// are never read, and a causal row stops at the first key past its position
// (positions increase along the block list).
#include "msa_common.h"

namespace msa {

template <typename T, int D>
__global__ __launch_bounds__(256) void msa_rowwise_kernel(KernelArgs a) {
  constexpr int E = D / 64;  // elements of head_dim per lane
  const WorkItem it = a.items[blockIdx.x];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = a.group;
  const int n_mrows = it.n_q * g;
  const T* __restrict__ K = (const T*)a.k;
  const T* __restrict__ V = (const T*)a.v;

  for (int mr = wave; mr < n_mrows; mr += 4) {
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
      const int valid = entry_valid(be);
      const int64_t phys = entry_block(be);
      const int64_t base = (phys * a.num_kv_heads + it.kv_head) * (int64_t)(kBlock * D);
      for (int s = 0; s < valid; ++s) {
        if (a.causal && be.pos0 + s > qp) break;
        const T* kr = K + base + s * D;
        const T* vr = V + base + s * D;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot += qv[e] * to_f32<T>(kr[lane * E + e]);
        const float x = wave_sum(dot) * a.scale_log2;
        const float mn = fmaxf(m, x);
        const float alpha = exp2f(m - mn);
        const float pr = exp2f(x - mn);
        l = l * alpha + pr;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + pr * to_f32<T>(vr[lane * E + e]);
        m = mn;
      }
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
}

template <typename T>
static int launch_rowwise(const KernelArgs& a, int head_dim, void* stream) {
  dim3 grid(a.n_items), block(256);
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
