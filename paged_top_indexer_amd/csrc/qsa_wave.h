// qsa_wave.h -- wave-level helpers shared by the HIP kernels (device code).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qsa {

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row_shr 1, 2,
// 4, 8 scan each row of 16 lanes, row_bcast 15 and 31 carry the row totals
// into the rows above.  All lanes must be active.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

}  // namespace qsa
