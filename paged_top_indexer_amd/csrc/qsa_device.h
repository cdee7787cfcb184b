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
// L2).  A row-indexed grid of `cols` columns (a row's chunks, attention
// splits or heads) places its work in one of two ways (Placement,
// qsa_launch.h):
//  - Cells dealt over the XCDs: cell_rows consecutive rows x one column form
//    a cell, cell c (row-major) goes to XCD c % 8, and its rows take
//    consecutive slots there.  A row's columns spread over the XCDs, so
//    every XCD gets an equal share of the work whatever the rows' lengths
//    and however few the rows; cells of several rows keep the same column of
//    neighbouring rows (a request's speculative-decode rows, which read the
//    same keys) in one L2.
//  - XCD groups: groups of kRowGroup consecutive rows, group g on XCD g % 8
//    with all its columns, so the kernels that work on one row meet on one
//    XCD and hand their data over through its L2.
// Workgroups mapped past the last row exit.
__device__ __forceinline__ int64_t row_on_xcd(int64_t xcd, int64_t s) {
  return kRowGroup * (kXcds * (s / kRowGroup) + xcd) + s % kRowGroup;
}

// (row, column) of workgroup b of a grid of grid_blocks(units, cols, pl)
// workgroups, `cols` per row.
struct RowCol {
  int64_t row, col;
};

__device__ __forceinline__ RowCol row_col_of_block(int64_t b, int64_t cols, Placement pl) {
  const int64_t xcd = b % kXcds;
  const int64_t slot = b / kXcds;
  if (pl.deal) {
    const int64_t cell = slot / pl.cell_rows * kXcds + xcd;
    return {cell / cols * pl.cell_rows + slot % pl.cell_rows, cell % cols};
  }
  return {row_on_xcd(xcd, slot / cols), slot % cols};
}

}  // namespace qsa
