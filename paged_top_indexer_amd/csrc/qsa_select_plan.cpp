// qsa_select_plan.cpp -- launch plan of the selection (host-only C++):
// chunk size, grid shape and the candidate area of the workspace.  Kept
// apart from the validation code because it fixes the selection kernels'
// memory traffic.
#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "qsa_launch.h"

namespace qsa {
namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Chunk size: the largest of 32/16/8/4/2/1 pages that still gives the chunk
// kernel about 1024 workgroups (4 per compute unit on 256 CUs, its
// occupancy), so long rows are split across the chip while short batches
// keep chunks small.  A table of at most 4 pages (512 blocks: every visible
// block is selected, no top-k) is one chunk per row whatever the batch, so
// short rows finish in the chunk kernel without a merge launch.
SelectPlan plan_select(int64_t rows, int64_t table_width, int group) {
  SelectPlan p;
  p.group = std::max(1, std::min(group, kMaxGroup));
  const int64_t groups = (rows + p.group - 1) / p.group;
  const int64_t w = table_width > 0 ? table_width : 1;
  int pages = max_chunk_pages(p.group);
  if (w * kPageSlots <= kTopKBlocks) {
    pages = (int)w;
  } else {
    while (pages > 1 && groups * ((w + pages - 1) / pages) < 1024) pages >>= 1;
  }
  p.chunk_pages = pages;
  p.chunks_per_row = (w + pages - 1) / pages;
  p.cand_cap = std::min<int64_t>(kTopKBlocks, (int64_t)pages * kPageSlots);
  if (rows == 0 || p.chunks_per_row == 1) {
    p.bytes = 0;
    return p;
  }
  size_t off = 0;
  const size_t cands = (size_t)rows * (size_t)p.chunks_per_row * (size_t)p.cand_cap;
  p.keys_off = off;
  off = align256(off + cands * sizeof(uint32_t));
  p.blocks_off = off;
  off = align256(off + cands * sizeof(uint32_t));
  p.bytes = off;
  return p;
}

}  // namespace qsa
