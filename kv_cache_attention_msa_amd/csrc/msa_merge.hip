// Log-sum-exp merge of KV-split partial results.
//
// A tile split over KV produces, per split i, the normalised output O_i of
// attention over that split's keys and its log-sum-exp L_i.  Over the union:
//   M = max_i L_i,  w_i = exp(L_i - M),  O = sum_i w_i O_i / sum_i w_i,
//   L = M + log(sum_i w_i).
// Splits are combined in index order (and the weights summed by a fixed
// butterfly), so the result is deterministic.  A row
// whose splits all saw no key (every L_i = -inf) gets O = 0, L = -inf.
#include "msa_common.h"

namespace msa {

// One wave per row: lane s takes split s's log-sum-exp (64 splits at a time),
// so the maximum and the weights come from one load per lane and wave
// reductions; then every lane accumulates its head_dim columns over the
// splits in index order, the weight of split j broadcast from lane j.
template <typename T, int D>
__global__ __launch_bounds__(256) void msa_merge_kernel(KernelArgs a) {
  constexpr int E = D / 64;
  const MergeItem mi = a.merges[blockIdx.x];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = a.group;
  const int ns = mi.n_splits;
  // work-group (x, y) merges rows 4 y .. 4 y + 3 of merge item x, one per wave
  {
    const int mr = 4 * blockIdx.y + wave;
    if (mr >= mi.n_mrows) return;
    const int row = mi.q_row0 + mr / g;
    const int head = mi.kv_head * g + mr % g;
    const int pr0 = mi.part_row0 + mr;   // split s of this row: partial row pr0 + s * n_mrows
    float M = kNegInf;
    for (int s0 = 0; s0 < ns; s0 += 64)
      if (s0 + lane < ns) M = fmaxf(M, a.part_lse[pr0 + (s0 + lane) * mi.n_mrows]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    if (M != kNegInf) {
      for (int s0 = 0; s0 < ns; s0 += 64) {
        const int s = s0 + lane;
        const float L = s < ns ? a.part_lse[pr0 + s * mi.n_mrows] : kNegInf;
        const float w = L == kNegInf ? 0.f : exp2f((L - M) * kLog2e);
        wsum += w;
        const int cnt = min(64, ns - s0);
        const float* po = a.part_o + (int64_t)(pr0 + s0 * mi.n_mrows) * D + lane * E;
        const int64_t step = (int64_t)mi.n_mrows * D;
        int j = 0;
        for (; j + 8 <= cnt; j += 8) {
          float v[8][E];
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = po[(j + u) * step + e];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float wj = __shfl(w, j + u, 64);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += wj > 0.f ? wj * v[u][e] : 0.f;
          }
        }
        for (; j < cnt; ++j) {
          const float wj = __shfl(w, j, 64);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] += wj > 0.f ? wj * po[j * step + e] : 0.f;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
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
  dim3 grid(a.n_merges, (a.max_mrows + 3) / 4), block(256);
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
