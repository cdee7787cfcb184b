// qsa_plan.cpp -- launch plans of the two stages (host-only C++): the
// selection's chunk size, grid shape and candidate area, and the attention's
// split length and partials.  Kept apart from the validation code because
// they fix the kernels' memory traffic.
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
// keep chunks small -- but no smaller than keeps a row's candidates
// (chunks x min(512, chunk)) within one merge batch of kFusedCands, where
// the largest chunk allows: every further batch of 8192 candidates costs
// the merge a whole radix select, more than a few rows' longer chunks cost
// the chunk kernel.  A table of at most 4 pages (512 blocks: every visible
// block is selected, no top-k) is one chunk per row whatever the batch, so
// short rows finish in the chunk kernel without a merge launch.
SelectPlan plan_select(int64_t rows, int64_t table_width, int group, bool big_ok) {
  SelectPlan p;
  p.group = std::max(1, std::min(group, kMaxGroup));
  const int64_t groups = (rows + p.group - 1) / p.group;
  const int64_t w = table_width > 0 ? table_width : 1;
  int pages = max_chunk_pages(p.group);
  // Long rows (4 or more 64-page chunks) of a batch that fills the chip with
  // them (512 workgroups, two per CU): 64-page chunks of 8-wave workgroups,
  // half the candidates of 32-page chunks for the kernel that finishes each
  // row.  (Rows of two such chunks lose more parallelism than they save.)
  const int big = max_chunk_pages(p.group, true);
  const int64_t big_chunks = (w + big - 1) / big;
  if (big_ok && p.group == 1 && big_chunks >= 4 && groups * big_chunks >= 512 &&
      big_chunks * kTopKBlocks <= kFusedCands) {
    p.big = true;
    pages = big;
  } else if (w * kPageSlots <= kTopKBlocks) {
    pages = (int)w;
  } else {
    while (pages > 1 && groups * ((w + pages - 1) / pages) < 1024) pages >>= 1;
    auto row_cands = [&](int pg) {
      return ((w + pg - 1) / pg) * std::min<int64_t>(kTopKBlocks, (int64_t)pg * kPageSlots);
    };
    while (pages < max_chunk_pages(p.group) && row_cands(pages) > kFusedCands) pages <<= 1;
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

// Splits: whole-CU workgroups (below) for 8 to 256 rows, and for fewer rows
// when asked (whole_cu: a decode step that selects inside the attention
// launch); otherwise 4-wave workgroups, enough splits for about one
// resident round of them over the batch (3 per CU on 256 CUs) in multiples
// of 64 index positions (each wave loads its indices 64 at a time) -- 33
// splits of 64 for a single row, one split per row from 768 rows up.
AttnPlan plan_attn(int64_t rows, bool whole_cu) {
  AttnPlan p;
  constexpr int64_t kResident = 768;
  const int64_t want =
      rows > 0 ? std::min<int64_t>(kMaxAttnSplits,
                                   std::max<int64_t>(1, (kResident + rows - 1) / rows))
               : 1;
  p.split_positions = 64 * (int)((kOutWidth + 64 * want - 1) / (64 * want));
  p.splits = (kOutWidth + p.split_positions - 1) / p.split_positions;
  // About one workgroup of kAttnRowWaves waves per CU (splits = 256 / rows,
  // at most 11 of 192 positions), each wave a whole number of 16-position
  // tiles; 256 rows take one workgroup per row and need no combine.  Below
  // 8 rows, 11 such workgroups per row (one tile per wave, 12 waves'
  // partials merged in LDS) are slower than 33 of 4 waves.
  constexpr int kUnit = 16 * kAttnRowWaves;
  if (rows > 0 && rows <= 256 && (whole_cu || rows >= 8)) {
    const int splits = (int)std::max<int64_t>(1, 256 / rows);
    p.waves = kAttnRowWaves;
    p.split_positions = kUnit * ((kOutWidth + splits * kUnit - 1) / (splits * kUnit));
    p.splits = (kOutWidth + p.split_positions - 1) / p.split_positions;
  }
  // (at most kMaxAttnSplits: the combine kernel holds every split's weight)
  if (rows == 0) return p;
  size_t off = 0;
  p.partial_off = off;
  off = align256(off + (size_t)rows * p.splits * kAttHeads * kAttDim * sizeof(float));
  p.stats_off = off;
  off = align256(off + (size_t)rows * p.splits * kAttHeads * 2 * sizeof(float));
  p.bytes = p.splits > 1 ? off : 0;
  return p;
}

// The selection runs inside the attention launch when every multi-chunk
// row's candidates fit the attention workgroup's LDS (at most kFusedCands)
// and the attention takes whole-CU workgroups (up to 256 rows).
DecodePlan plan_decode(int64_t rows, int64_t table_width, int group) {
  DecodePlan d;
  d.select = plan_select(rows, table_width, group, true);
  const bool fusable = d.select.chunks_per_row > 1 &&
                       d.select.chunks_per_row * d.select.cand_cap <= kFusedCands;
  d.attn = plan_attn(rows, fusable);
  d.fused = fusable && d.attn.waves == kAttnRowWaves;
  d.attn_off = align256(d.select.bytes);
  d.bytes = d.attn_off + d.attn.bytes;
  return d;
}

}  // namespace qsa
