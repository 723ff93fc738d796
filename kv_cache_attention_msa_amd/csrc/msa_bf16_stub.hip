// Temporary bf16 launchers: route prefill and decode items to the row-at-a-time kernel.
#include "msa_common.h"

namespace msa {

int launch_rowwise_bf16(const KernelArgs& a, int head_dim, void* stream);

int launch_prefill(const KernelArgs& a, int head_dim, void* stream) {
  return launch_rowwise_bf16(a, head_dim, stream);
}
int launch_decode(const KernelArgs& a, int head_dim, void* stream) {
  return launch_rowwise_bf16(a, head_dim, stream);
}

}  // namespace msa
