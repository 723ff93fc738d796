// Attainable-rate probes (see include/msa_peaks.h): a streaming HBM read and
// a bf16 MFMA issue loop.  Measurement tooling for the benchmark only.
#include <hip/hip_runtime.h>

#include <utility>
#include <vector>

#include "msa_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, size_t n, uint32_t* out) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)(p + i));
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) out[0] = acc;  // keeps the loads live; practically never taken
}

// One wave per 4 KiB block: 4 loads of 16 bytes per lane.
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ pool, const int32_t* __restrict__ ids,
                                                     int32_t blocks, uint32_t* out) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= blocks) return;
  const int lane = threadIdx.x & 63;
  const u32x4_t* b = (const u32x4_t*)(pool + (size_t)ids[w] * 256);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t v = __builtin_nontemporal_load(b + j * 64 + lane);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) out[0] = acc;  // keeps the loads live; practically never taken
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint4 v = src[i];
    __builtin_nontemporal_store(v.x, &dst[i].x);
    __builtin_nontemporal_store(v.y, &dst[i].y);
    __builtin_nontemporal_store(v.z, &dst[i].z);
    __builtin_nontemporal_store(v.w, &dst[i].w);
  }
}

__global__ __launch_bounds__(256) void mfma_kernel(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  f32x16 c0 = (f32x16){0}, c1 = (f32x16){0}, c2 = (f32x16){0}, c3 = (f32x16){0};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const float s = c0[0] + c1[5] + c2[10] + c3[15];
  if (s == 1234.5f) out[threadIdx.x] = s;
}

#define PK_HIP(x)                      \
  do {                                 \
    if ((x) != hipSuccess) return -5;  \
  } while (0)

}  // namespace

extern "C" int msa_peak_hbm_read(size_t bytes, int iters, double* gbps) {
  if (!gbps || bytes == 0 || bytes % 16 || iters <= 0) return -1;
  void* p = nullptr;
  uint32_t* out = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -5;
  if (hipMalloc(&p, bytes) == hipSuccess && hipMalloc(&out, 64) == hipSuccess &&
      hipMemset(p, 1, bytes) == hipSuccess && hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess &&
      hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    int dev = 0, cus = 256;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const dim3 grid(8 * cus);
    const size_t n = bytes / 16;
    hipLaunchKernelGGL(read_kernel, grid, dim3(256), 0, s, (const uint4*)p, n, out);
    (void)hipEventRecord(e0, s);
    for (int i = 0; i < iters; ++i) hipLaunchKernelGGL(read_kernel, grid, dim3(256), 0, s, (const uint4*)p, n, out);
    (void)hipEventRecord(e1, s);
    float ms = 0.f;
    if (hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f) {
      *gbps = (double)bytes * iters / (ms * 1e-3) / 1e9;
      rc = 0;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (s) (void)hipStreamDestroy(s);
  if (out) (void)hipFree(out);
  if (p) (void)hipFree(p);
  return rc;
}

extern "C" int msa_peak_hbm_copy(size_t bytes, int iters, double* gbps) {
  if (!gbps || bytes == 0 || bytes % 16 || iters <= 0) return -1;
  void *src = nullptr, *dst = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -5;
  if (hipMalloc(&src, bytes) == hipSuccess && hipMalloc(&dst, bytes) == hipSuccess &&
      hipMemset(src, 1, bytes) == hipSuccess && hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess &&
      hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    int dev = 0, cus = 256;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const dim3 grid(8 * cus);
    const size_t n = bytes / 16;
    hipLaunchKernelGGL(copy_kernel, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, n);
    (void)hipEventRecord(e0, s);
    for (int i = 0; i < iters; ++i) hipLaunchKernelGGL(copy_kernel, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, n);
    (void)hipEventRecord(e1, s);
    float ms = 0.f;
    if (hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f) {
      *gbps = 2.0 * (double)bytes * iters / (ms * 1e-3) / 1e9;
      rc = 0;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (s) (void)hipStreamDestroy(s);
  if (dst) (void)hipFree(dst);
  if (src) (void)hipFree(src);
  return rc;
}

extern "C" int msa_peak_hbm_gather(int32_t blocks, int iters, double* gbps) {
  if (!gbps || blocks <= 0 || iters <= 0) return -1;
  const size_t pool_blocks = 2 * (size_t)blocks;
  std::vector<int32_t> ids(pool_blocks);
  for (size_t i = 0; i < pool_blocks; ++i) ids[i] = (int32_t)i;
  uint64_t x = 0x2545F4914F6CDD1Dull;  // xorshift64*, fixed seed
  for (size_t i = pool_blocks - 1; i > 0; --i) {
    x ^= x >> 12; x ^= x << 25; x ^= x >> 27;
    const size_t j = (size_t)((x * 0x2545F4914F6CDD1Dull) % (i + 1));
    std::swap(ids[i], ids[j]);
  }
  void* pool = nullptr;
  int32_t* d_ids = nullptr;
  uint32_t* out = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -5;
  const size_t bytes = pool_blocks * 4096;
  if (hipMalloc(&pool, bytes) == hipSuccess && hipMalloc(&d_ids, blocks * sizeof(int32_t)) == hipSuccess &&
      hipMalloc(&out, 64) == hipSuccess && hipMemset(pool, 1, bytes) == hipSuccess &&
      hipMemcpy(d_ids, ids.data(), blocks * sizeof(int32_t), hipMemcpyHostToDevice) == hipSuccess &&
      hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess && hipEventCreate(&e0) == hipSuccess &&
      hipEventCreate(&e1) == hipSuccess) {
    const dim3 grid((unsigned)((blocks + 3) / 4));
    hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, (const uint4*)pool, d_ids, blocks, out);
    (void)hipEventRecord(e0, s);
    for (int i = 0; i < iters; ++i)
      hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, (const uint4*)pool, d_ids, blocks, out);
    (void)hipEventRecord(e1, s);
    float ms = 0.f;
    if (hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f) {
      *gbps = (double)blocks * 4096.0 * iters / (ms * 1e-3) / 1e9;
      rc = 0;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (s) (void)hipStreamDestroy(s);
  if (out) (void)hipFree(out);
  if (d_ids) (void)hipFree(d_ids);
  if (pool) (void)hipFree(pool);
  return rc;
}

extern "C" int msa_peak_mfma_bf16(int iters, double* tflops) {
  if (!tflops || iters <= 0) return -1;
  float* out = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -5;
  if (hipMalloc(&out, 4096) == hipSuccess && hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess &&
      hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    int dev = 0, cus = 256;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int grid = 8 * cus;  // 8 work-groups of 4 waves per CU
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, s, out, 10);
    (void)hipEventRecord(e0, s);
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, s, out, iters);
    (void)hipEventRecord(e1, s);
    float ms = 0.f;
    if (hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f) {
      const double flops = (double)grid * 4 * iters * 4 * (2.0 * 32 * 32 * 16);
      *tflops = flops / (ms * 1e-3) / 1e12;
      rc = 0;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (s) (void)hipStreamDestroy(s);
  if (out) (void)hipFree(out);
  return rc;
}
