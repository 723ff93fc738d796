// Plan upload: the host packs each call's plan into pinned, device-mapped
// memory and this kernel copies it into the pool's device plan buffer on the
// caller's stream, ahead of the attention kernels that read it.  Staying on
// the caller's queue avoids a DMA-engine-to-compute-queue hand-off per call.
#include "msa_common.h"

namespace msa {

__global__ __launch_bounds__(256) void msa_upload_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

int launch_upload(const void* src, void* dst, size_t bytes, void* stream) {
  const size_t n = bytes / 16;
  if (n == 0) return 0;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(msa_upload_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, n);
  return (int)hipGetLastError();
}

}  // namespace msa
