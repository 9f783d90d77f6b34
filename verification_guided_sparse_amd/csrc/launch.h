// launch.h -- host-side launchers of the attention kernels.  Each kernel
// family is instantiated in its own translation unit (k_*.hip), so that the
// library builds in parallel; the host planning in vegas_attn.hip calls these.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_common.h"

#ifndef VG_VERIFY_PF
#define VG_VERIFY_PF 2   // tiles in flight per wave, D = 128
#endif
#ifndef VG_VERIFY_PF64
#define VG_VERIFY_PF64 1  // D = 64: one tile in flight, two workgroups per CU
#endif
#ifndef VG_SPARSE_PF
#define VG_SPARSE_PF 1   // tiles in flight per wave, sparse draft
#endif

// Tiles in flight per wave of the verify kernel: at D = 128 two (one when 3 or
// 4 row tiles leave no registers for a second); at D = 64 one with two
// workgroups per CU, and two when 4 row tiles make the merge area too large
// for a second workgroup (one tile per wave in flight on one workgroup per
// CU is too few bytes in flight to stream HBM).
constexpr int verify_pf(int D, int NT) {
  return D == 128 ? (NT <= 2 ? VG_VERIFY_PF : 1) : (NT <= 3 ? VG_VERIFY_PF64 : 2);
}

namespace vg {

// grid = one workgroup per piece of the plan, kThreads threads each
// share_entries: the most entries one verify workgroup's share can hold
void launch_mfma128_verify(int nt, const AttnArgs &a, dim3 grid, hipStream_t st, long long share_entries);
void launch_mfma128_sparse(int nt, const AttnArgs &a, dim3 grid, hipStream_t st);
void launch_mfma64_verify(int nt, const AttnArgs &a, dim3 grid, hipStream_t st);
void launch_mfma64_sparse(int nt, const AttnArgs &a, dim3 grid, hipStream_t st);
void launch_valu_f32128(int mr, const AttnArgs &a, dim3 grid, hipStream_t st);
void launch_valu_f3264(int mr, const AttnArgs &a, dim3 grid, hipStream_t st);
void launch_valu_bf16128(int mr, const AttnArgs &a, dim3 grid, hipStream_t st);
void launch_valu_bf1664(int mr, const AttnArgs &a, dim3 grid, hipStream_t st);

}  // namespace vg
