// k_valu_f32128.hip -- instantiations of the vector-ALU attention kernel for
// f32 caches at D = 128, row blocks of 16, 32 or 64.
#include "launch.h"
#include "attn_valu.h"

namespace vg {

void launch_valu_f32128(int mr, const AttnArgs &a, dim3 grid, hipStream_t st) {
  switch (mr) {
    case 16: hipLaunchKernelGGL((attn_valu_kernel<float, 128, 16>), grid, dim3(kThreads), 0, st, a); break;
    case 32: hipLaunchKernelGGL((attn_valu_kernel<float, 128, 32>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((attn_valu_kernel<float, 128, 64>), grid, dim3(kThreads), 0, st, a); break;
  }
}

}  // namespace vg
