// Decode kernel for bf16 pools: one work item (a handful of (query row, q
// head) pairs of one sequence and kv head against a run of KV blocks) per
// work-group; the work itself is decode_item (msa_decode_item.h).
#include "msa_decode_item.h"

namespace msa {
namespace {

using dec::kDecodeThreads;

template <int D, int NM>
__global__ __launch_bounds__(kDecodeThreads, 3) void msa_decode_kernel(KernelArgs a) {
  __shared__ dec::VRing<D> vr0;
  __shared__ dec::VRing<D> vr1;
  dec::decode_item<D, NM>(a, a.items[blockIdx.x], vr0, vr1);
}

template <int D>
int launch_d(const KernelArgs& a, void* stream) {
  dim3 grid(a.n_items), block(kDecodeThreads);
  hipStream_t s = (hipStream_t)stream;
  if (a.max_mrows > kDecodeMRows) return (int)hipErrorInvalidValue;
  if (a.max_mrows <= 4) hipLaunchKernelGGL((msa_decode_kernel<D, 4>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((msa_decode_kernel<D, 8>), grid, block, 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_decode(const KernelArgs& a, int head_dim, void* stream) {
  return head_dim == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace msa
