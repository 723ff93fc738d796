// Plan upload: the host packs each call's plan into pinned, device-mapped
// memory and this kernel copies it into the pool's device plan buffer on the
// caller's stream, ahead of the attention kernels that read it.  Staying on
// the caller's queue avoids a DMA-engine-to-compute-queue hand-off per call.
// On the way it replaces each block-list entry's block-table index by the
// pool block id found there, so the attention kernels read block ids
// directly (one dependent load less per block).
#include "msa_common.h"

namespace msa {

__device__ __forceinline__ uint32_t resolve(uint32_t bt_valid, const int32_t* __restrict__ bt, int32_t nb) {
  const uint32_t mask = (1u << kBtIndexBits) - 1u;
  int32_t id = bt[bt_valid & mask];
  id = min(max(id, 0), nb - 1);
  return (uint32_t)id | (bt_valid & ~mask);
}

// The block list sits at the start of the plan: 16-byte chunk i holds
// entries 2i and 2i+1 (x/y and z/w).
__global__ __launch_bounds__(256) void msa_upload_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          size_t n, int32_t n_blocks,
                                                          const int32_t* __restrict__ block_table,
                                                          int32_t num_blocks) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint4 u = src[i];
    if ((int64_t)(2 * i) < n_blocks) u.x = resolve(u.x, block_table, num_blocks);
    if ((int64_t)(2 * i + 1) < n_blocks) u.z = resolve(u.z, block_table, num_blocks);
    dst[i] = u;
  }
}

// Optional block-id check: counts the entries of a host-packed block list
// whose block-table entry holds an id outside [0, num_blocks), and keeps the
// smallest such block-table index.  result[0] must start at 0 and result[1]
// at INT32_MAX.
__global__ __launch_bounds__(256) void msa_check_ids_kernel(const BlockEntry* __restrict__ src, int32_t n_blocks,
                                                             const int32_t* __restrict__ block_table,
                                                             int32_t num_blocks, int32_t* result) {
  const uint32_t mask = (1u << kBtIndexBits) - 1u;
  for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n_blocks; i += gridDim.x * blockDim.x) {
    const int32_t idx = (int32_t)((uint32_t)src[i].bt_valid & mask);
    const int32_t id = block_table[idx];
    if (id < 0 || id >= num_blocks) {
      atomicAdd(&result[0], 1);
      atomicMin(&result[1], idx);
    }
  }
}

int launch_check_ids(const void* src, int32_t n_blocks, const int32_t* block_table, int32_t num_blocks,
                     int32_t* result, void* stream) {
  if (n_blocks <= 0) return 0;
  const int blocks = std::min((n_blocks + 255) / 256, 1024);
  hipLaunchKernelGGL(msa_check_ids_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const BlockEntry*)src,
                     n_blocks, block_table, num_blocks, result);
  return (int)hipGetLastError();
}

int launch_upload(const void* src, void* dst, size_t bytes, int32_t n_blocks, const int32_t* block_table,
                  int32_t num_blocks, void* stream) {
  const size_t n = bytes / 16;
  if (n == 0) return 0;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(msa_upload_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, n, n_blocks, block_table, num_blocks);
  return (int)hipGetLastError();
}

}  // namespace msa
