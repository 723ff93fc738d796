// Log-sum-exp merge of KV-split partial results.
//
// A tile split over KV produces, per split i, the normalised output O_i of
// attention over that split's keys and its log-sum-exp L_i.  Over the union:
//   M = max_i L_i,  w_i = exp(L_i - M),  O = sum_i w_i O_i / sum_i w_i,
//   L = M + log(sum_i w_i).
// Splits are combined in index order, so the result is deterministic.  A row
// whose splits all saw no key (every L_i = -inf) gets O = 0, L = -inf.
#include "msa_common.h"

namespace msa {

template <typename T, int D>
__global__ __launch_bounds__(256) void msa_merge_kernel(KernelArgs a) {
  constexpr int E = D / 64;
  const MergeItem mi = a.merges[blockIdx.x];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = a.group;
  for (int mr = wave; mr < mi.n_mrows; mr += 4) {
    const int row = mi.q_row0 + mr / g;
    const int head = mi.kv_head * g + mr % g;
    float M = kNegInf;
    for (int s = 0; s < mi.n_splits; ++s) M = fmaxf(M, a.part_lse[mi.part_row0 + s * mi.n_mrows + mr]);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    if (M != kNegInf) {
      for (int s = 0; s < mi.n_splits; ++s) {
        const int pr = mi.part_row0 + s * mi.n_mrows + mr;
        const float w = exp2f((a.part_lse[pr] - M) * kLog2e);
        wsum += w;
        const float* po = a.part_o + (int64_t)pr * D;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * po[lane * E + e];
      }
    }
    const bool any = wsum > 0.f;
    const float inv = any ? 1.f / wsum : 0.f;
    T* orow = (T*)a.out + ((int64_t)row * a.num_q_heads + head) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[lane * E + e] = from_f32<T>(acc[e] * inv);
    if (a.lse && lane == 0) a.lse[(int64_t)row * a.num_q_heads + head] = any ? M + logf(wsum) : kNegInf;
  }
}

int launch_merge(const KernelArgs& a, int head_dim, int dtype, void* stream) {
  dim3 grid(a.n_merges), block(256);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MSA_FP32) {
    if (head_dim == 128) hipLaunchKernelGGL((msa_merge_kernel<float, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((msa_merge_kernel<float, 64>), grid, block, 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((msa_merge_kernel<bf16_t, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((msa_merge_kernel<bf16_t, 64>), grid, block, 0, s, a);
  }
  return (int)hipGetLastError();
}

}  // namespace msa
