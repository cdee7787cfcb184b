// qsa_device.h -- device helpers shared by the HIP kernels: a DPP wave scan
// and the XCD-aware placement of row-indexed grids.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_launch.h"

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

// Workgroups are dealt to the XCDs round-robin by id (each XCD has its own
// L2).  Row-indexed grids place rows in groups of kRowGroup consecutive rows
// (group g on XCD g % 8), the same way in every kernel of the path: the
// kernels that work on one row (chunks, merge, attention splits, combine)
// then meet on one XCD and hand their data over through its L2, and the
// rows of one request (consecutive for speculative-decode and prefill rows)
// read the same keys through the same L2.  Workgroup b is the (b / 8)-th
// workgroup of XCD b % 8; that XCD's s-th row is row_on_xcd(b % 8, s).
// Grids are padded to whole groups on all XCDs; workgroups mapped past the
// last row exit.
// (kXcds, kRowGroup and padded_rows are in qsa_launch.h, shared with the
// host code that sizes the grids.)
__device__ __forceinline__ int64_t row_on_xcd(int64_t xcd, int64_t s) {
  return kRowGroup * (kXcds * (s / kRowGroup) + xcd) + s % kRowGroup;
}

// (row, column) of workgroup b of a grid with `cols` workgroups per row.
struct RowCol {
  int64_t row, col;
};

__device__ __forceinline__ RowCol row_col_of_block(int64_t b, int64_t cols) {
  const int64_t slot = b / kXcds;
  return {row_on_xcd(b % kXcds, slot / cols), slot % cols};
}

}  // namespace qsa
