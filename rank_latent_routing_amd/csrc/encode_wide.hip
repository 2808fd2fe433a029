// The 8-wave, 32-feature instantiation of the split-token encoder
// (encode_kernel.hpp): 256 latents per workgroup, the kernel of the
// large-latent workloads.  This file alone is compiled with LLVM's
// iterative ILP scheduling strategy for AMDGPU
// (-amdgpu-sched-strategy=iterative-ilp): with it this kernel ran 2.5-3.4 %
// faster, while the narrower instantiations would spill.
#include "encode_kernel.hpp"

namespace flare {

hipError_t launch_encode_bf16_wide(const EncodeParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((encode_bf16_kernel<32, 8>), grid, dim3(64 * 8), 0, st, p);
  return hipGetLastError();
}

}  // namespace flare
