// KV write (recompute-scatter): copies freshly computed K/V rows into the pool
// blocks that their segments name, so that the attention kernels read them as
// ordinary cache blocks.
//
// The source is the row-major output of a K/V projection, [rows][H_kv][d]; a
// (block, kv head) tile of the pool is 16 slots x d contiguous elements.  One
// wave moves one tile of K and the same tile of V: each 16-byte chunk of the
// tile comes from one token row of the same head (a 256-byte run for bf16 and
// d = 128), so both the loads and the stores are whole, aligned 16-byte
// accesses and every instruction covers four full 256-byte rows.  All of a
// lane's loads are issued before its stores.  The stores are non-temporal:
// the written blocks are not read again by this call, and streaming them past
// the caches keeps those for the source rows (measured: 98 -> 56 us warm on
// 367 MB, and at the rate of a plain non-temporal copy when cold).  Slots
// past a block's valid count are neither read nor written.  HBM-bound: each
// fresh byte is read once and written once.
#include "msa_common.h"

namespace msa {

__device__ __forceinline__ void store_stream(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(v.x, &p->x);
  __builtin_nontemporal_store(v.y, &p->y);
  __builtin_nontemporal_store(v.z, &p->z);
  __builtin_nontemporal_store(v.w, &p->w);
}

template <int ROW>  // bytes of one (token, head) row: head_dim * element size
__global__ __launch_bounds__(256) void msa_write_kernel(WriteArgs a) {
  constexpr int kChunks = ROW / 16;              // 16-byte chunks per row
  constexpr int kPerLane = kBlock * kChunks / 64;
  static_assert(kPerLane * 64 == kBlock * kChunks, "tile must split evenly over a wave");
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= a.n_entries * a.num_kv_heads) return;
  const int lane = threadIdx.x & 63;
  const int e = task / a.num_kv_heads;
  const int h = task - e * a.num_kv_heads;
  const BlockEntry be = a.blocks[e];
  const int blk = entry_block(be);
  const int valid = entry_valid(be);
  const size_t pitch = (size_t)a.num_kv_heads * ROW;  // bytes per source token
  const size_t src0 = (size_t)(uint32_t)be.pos0 * pitch + (size_t)h * ROW;
  const size_t dst0 = ((size_t)blk * a.num_kv_heads + h) * (kBlock * ROW);
  const char* ks = (const char*)a.k_src + src0;
  const char* vs = (const char*)a.v_src + src0;
  char* kd = (char*)a.k + dst0;
  char* vd = (char*)a.v + dst0;
  uint4 kr[kPerLane], vr[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int c = j * 64 + lane;
    const int slot = c / kChunks;
    const int col = c % kChunks;
    if (slot < valid) {
      kr[j] = *(const uint4*)(ks + slot * pitch + col * 16);
      vr[j] = *(const uint4*)(vs + slot * pitch + col * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int c = j * 64 + lane;
    if (c / kChunks < valid) {
      store_stream((uint4*)(kd + c * 16), kr[j]);
      store_stream((uint4*)(vd + c * 16), vr[j]);
    }
  }
}

int launch_write(const WriteArgs& a, int row_bytes, void* stream) {
  const int64_t tasks = (int64_t)a.n_entries * a.num_kv_heads;
  if (tasks <= 0) return 0;
  dim3 grid((unsigned)((tasks + 3) / 4)), block(256);
  hipStream_t s = (hipStream_t)stream;
  switch (row_bytes) {
    case 128: hipLaunchKernelGGL(msa_write_kernel<128>, grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(msa_write_kernel<256>, grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL(msa_write_kernel<512>, grid, block, 0, s, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace msa
