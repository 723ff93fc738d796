// Fixed device scratch for msa_forward_noalloc, the entry point for callers
// that cannot allocate device memory.
//
// The scratch is one file-scope __device__ array, so every GPU the library
// runs on holds its own copy from module load until the process ends.  Host
// code never uses the array's name as an address (on the host it only names
// a stand-in symbol): the device address of each GPU's copy is looked up once
// per device, with that device current, through hipGetSymbolAddress, and
// only that address is handed to copies and kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "msa_internal.h"

namespace msa {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int scratch_address(int device, void** ptr, std::string& err) {
  if (device < 0 || device >= kMaxDevices) {
    err = "device ordinal out of range for the fixed scratch";
    return MSA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[device]) {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != device) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != device) (void)hipSetDevice(prev);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      err = std::string("hipGetSymbolAddress of the fixed scratch failed: ") + hipGetErrorString(e);
      return MSA_ERR_HIP;
    }
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return MSA_OK;
}

}  // namespace msa
