// One block-size specialisation of the selection kernels: the build compiles
// this file once per supported block size with -DDSA_BS=<size> (0 stands for
// every other size), so the specialisations compile in parallel.
#include "dsa_kernels.hpp"

#ifndef DSA_BS
#error "DSA_BS must be defined (a block size in {0, 1, 2, 4, 8, 16, 32, 64})"
#endif

namespace dsa {

template <>
void launch<DSA_BS>(Kernel k, unsigned grid, const Params& p, hipStream_t stream) {
  switch (k) {
    case Kernel::Fused:
      hipLaunchKernelGGL(k_fused<DSA_BS>, dim3(grid), dim3(NT), 0, stream, p);
      break;
    case Kernel::FusedBalanced:
      hipLaunchKernelGGL(k_fused_bal<DSA_BS>, dim3(grid), dim3(NT), 0, stream, p);
      break;
    case Kernel::Scores:
      hipLaunchKernelGGL(k_scores<DSA_BS>, dim3(grid), dim3(NT), 0, stream, p);
      break;
    case Kernel::Mask:
      hipLaunchKernelGGL(k_mask<DSA_BS>, dim3(grid), dim3(NT), 0, stream, p);
      break;
    case Kernel::TopkTokens:
      hipLaunchKernelGGL(k_topk_tokens<DSA_BS>, dim3(grid), dim3(NT), 0, stream, p);
      break;
  }
}

}  // namespace dsa
