// k_valu_bf1664.hip -- instantiations of the vector-ALU attention kernel for
// bf16 caches at D = 64, row blocks of 16, 32 or 64.
#include "launch.h"
#include "attn_valu.h"

namespace vg {

void launch_valu_bf1664(int mr, const AttnArgs &a, dim3 grid, hipStream_t st) {
  switch (mr) {
    case 16: hipLaunchKernelGGL((attn_valu_kernel<uint16_t, 64, 16>), grid, dim3(kThreads), 0, st, a); break;
    case 32: hipLaunchKernelGGL((attn_valu_kernel<uint16_t, 64, 32>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((attn_valu_kernel<uint16_t, 64, 64>), grid, dim3(kThreads), 0, st, a); break;
  }
}

}  // namespace vg
