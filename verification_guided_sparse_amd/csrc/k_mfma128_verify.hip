// k_mfma128_verify.hip -- instantiations of the matrix-core attention kernel,
// D = 128, verify mode, for 1..4 row tiles.
#include "launch.h"
#include "attn_mfma.h"

namespace vg {

template <int NT>
static void launch_nt(const AttnArgs &a, dim3 grid, hipStream_t st, bool long_chunks) {
  constexpr int PF = verify_pf(128, NT);
  if (a.logits)
    hipLaunchKernelGGL((attn_mfma_kernel<128, NT, PF, false, true>), grid, dim3(kThreads), 0, st, a);
  else if (long_chunks)
    hipLaunchKernelGGL((attn_mfma_kernel<128, NT, PF, false, false, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<128, NT, PF, false>), grid, dim3(kThreads), 0, st, a);
}

void launch_mfma128_verify(int nt, const AttnArgs &a, dim3 grid, hipStream_t st, long long share_entries) {
  const bool long_chunks = share_entries > kVerifyChunk;  // shares of more than one chunk
  switch (nt) {
    case 1: launch_nt<1>(a, grid, st, long_chunks); break;
    case 2: launch_nt<2>(a, grid, st, long_chunks); break;
    case 3: launch_nt<3>(a, grid, st, long_chunks); break;
    default: launch_nt<4>(a, grid, st, long_chunks); break;
  }
}

}  // namespace vg
