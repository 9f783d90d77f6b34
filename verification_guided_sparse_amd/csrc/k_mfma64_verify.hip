// k_mfma64_verify.hip -- instantiations of the matrix-core attention kernel,
// D = 64, verify mode, for 1..4 row tiles.
#include "launch.h"
#include "attn_mfma.h"

namespace vg {

template <int NT>
static void launch_nt(const AttnArgs &a, dim3 grid, hipStream_t st) {
  if (a.logits)
    hipLaunchKernelGGL((attn_mfma_kernel<64, NT, verify_pf(64, NT), false, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<64, NT, verify_pf(64, NT), false>), grid, dim3(kThreads), 0, st, a);
}

void launch_mfma64_verify(int nt, const AttnArgs &a, dim3 grid, hipStream_t st) {
  switch (nt) {
    case 1: launch_nt<1>(a, grid, st); break;
    case 2: launch_nt<2>(a, grid, st); break;
    case 3: launch_nt<3>(a, grid, st); break;
    default: launch_nt<4>(a, grid, st); break;
  }
}

}  // namespace vg
