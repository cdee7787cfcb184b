// qsa_launch.h -- internal interface between the host-side validation and
// planning code (qsa_capi.cpp, plain C++) and the HIP kernels (*.hip).
// Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

namespace qsa {

// Fixed contract: 512 blocks of 4 tokens plus a tail of at most 3 tokens.
constexpr int kTopKBlocks = 512;
constexpr int kRatio = 4;
constexpr int kOutWidth = 2051;
constexpr int kPageSlots = 128;
constexpr int kSelHeads = 4;
constexpr int kSelDim = 128;
constexpr int kAttHeads = 3;
constexpr int kAttDim = 256;
constexpr int kKvRow = 512;
constexpr int kKvPageTokens = 512;

// Row-indexed grids place kRowGroup consecutive rows together on the kXcds
// XCDs (see qsa_device.h).  A dispatch holds fewer than 2^32 work-items
// (workgroups x threads per workgroup).
constexpr int kXcds = 8;
constexpr int kRowGroup = 4;
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;

// Threads per workgroup of each kernel (the host checks grid sizes with
// them).
constexpr int kChunkThreads = 256;
constexpr int kChunkBigThreads = 512;  // 64-page chunks (SelectPlan::big)
constexpr int kMergeThreads = 768;
constexpr int kAttnThreads = 256;
constexpr int kCombineThreads = 256;

// Attention splits per row: plan_attn never plans more than kMaxAttnSplits,
// and the combine kernel keeps one weight per split in LDS.
constexpr int kMaxAttnSplits = (kOutWidth + 63) / 64;  // 33 splits of 64 positions
constexpr int kCombineMaxSplits = 64;
// Waves of a workgroup that takes a whole row of index positions (3 per
// SIMD, the split kernel's occupancy).
constexpr int kAttnRowWaves = 12;
static_assert(kMaxAttnSplits <= kCombineMaxSplits, "combine holds every split's weight");

// Bytes of the fixed device scratch of the no-allocation decode step (one
// copy per GPU, held until the process ends).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;

constexpr int64_t padded_rows(int64_t rows) {
  return (rows + kXcds * kRowGroup - 1) / (kXcds * kRowGroup) * (kXcds * kRowGroup);
}

// Placement of a row-indexed grid on the XCDs (see qsa_device.h): cells of
// `cell_rows` consecutive rows x one column dealt round-robin (deal), or
// XCD groups of kRowGroup rows with all their columns.
struct Placement {
  bool deal;
  int cell_rows;
};

// The chunk kernel over `units` rows, or runs of `group` rows of one
// request: cells of kRowGroup rows (neighbouring rows of a request read the
// same keys), except a single row (its chunk, merge, attention and combine
// workgroups then share one L2) and 32 or more runs (a prefill request's
// runs read their keys through one L2), placed by XCD groups.
constexpr Placement chunk_placement(int64_t units, int group) {
  return {units > 1 && (group == 1 || units < kXcds * kRowGroup), kRowGroup};
}

// The attention and combine kernels over `rows` rows: cells of one row, so
// that every XCD gets an equal share of the splits -- except a single row,
// and rows that fill whole groups on every XCD (a multiple of 32 rows),
// placed by XCD groups (measured 1-1.3% faster there than dealt).
constexpr Placement attn_placement(int64_t rows) {
  return {rows > 1 && rows % (kXcds * kRowGroup) != 0, 1};
}

// Workgroups of a row-indexed grid of `cols` columns over `units` rows:
// whole rounds of cells on all XCDs, or whole XCD groups.  Never more than
// padded_rows(units) * cols.
constexpr int64_t grid_blocks(int64_t units, int64_t cols, Placement pl) {
  if (!pl.deal) return padded_rows(units) * cols;
  const int64_t cells = (units + pl.cell_rows - 1) / pl.cell_rows * cols;
  return (cells + kXcds - 1) / kXcds * (kXcds * pl.cell_rows);
}

// Query rows scored together against one key stream: 4 rows x 4 heads fill
// the 16 rows of the MFMA's A operand.
constexpr int kMaxGroup = 4;

// Largest chunk (in cache pages) for groups of `group` rows: the chunk
// kernel keeps group * chunk_pages * 128 scores in LDS (at most 4096 with 4
// waves, 8192 with the 8 of a big plan), and a group's rows are selected
// one per wave from at most 1024 scores each.
constexpr int max_chunk_pages(int group, bool big = false) {
  return group <= 1 ? (big ? 64 : 32) : 8;
}

// Launch plan of the selection.  A row's visible blocks are cut into chunks
// of `chunk_pages` cache pages; one workgroup of the chunk kernel scores one
// chunk for a group of `group` consecutive query rows (reading each of the
// group's requests' keys once) and keeps each row's best min(512, chunk)
// blocks (a row with a single chunk is finished there).  The merge kernel
// then takes each multi-chunk row's candidates to the final top-512.
struct SelectPlan {
  int group = 1;               // query rows per chunk workgroup (1..4)
  int chunk_pages = 1;         // pages per chunk (1, 2, 4, 8, 16 or 32; or the
                               // whole table when it has at most 4 pages)
  int64_t chunks_per_row = 1;  // grid columns per row (ceil(W / chunk_pages))
  int64_t cand_cap = 0;        // candidate slots per chunk: min(512, 128*chunk_pages)
  bool big = false;            // 64-page chunks of kChunkBigThreads threads
  size_t keys_off = 0;         // byte offsets inside the workspace
  size_t blocks_off = 0;
  size_t bytes = 0;            // total workspace bytes (0 = none needed)
};

// big_ok: a selection from keys (not paged logits, not a logits matrix),
// which may take 64-page chunks of 8-wave workgroups.
SelectPlan plan_select(int64_t rows, int64_t table_width, int group = 1, bool big_ok = false);

// Launch plan of the attention kernel: `splits` workgroups per row, each
// covering `split_positions` index positions with `waves` waves (tiles of
// 16 positions): kAttnRowWaves (about one workgroup per CU) for 8 to 256
// rows, or from one row with whole_cu; 4 waves per split otherwise.
struct AttnPlan {
  int split_positions = 128;
  int splits = 1;
  int waves = 4;
  size_t partial_off = 0;  // [rows][splits][3][256] fp32 unnormalised outputs
  size_t stats_off = 0;    // [rows][splits][3][2] fp32 (running max, sum)
  size_t bytes = 0;
};

AttnPlan plan_attn(int64_t rows, bool whole_cu = false);

// Plans of the decode step: the selection's, the attention's, whether the
// attention launch finishes the selection (no merge launch), and the
// workspace (the selection's at 0, the attention's at attn_off).
struct DecodePlan {
  SelectPlan select;
  AttnPlan attn;
  bool fused = false;
  size_t attn_off = 0;
  size_t bytes = 0;
};

DecodePlan plan_decode(int64_t rows, int64_t table_width, int group);

// Arguments of the selection family.  Scores come from fp16 keys (kcache),
// e4m3 keys (kcodes + kscale) or a logits matrix (logits_in); they are
// selected (launch_select) or written out as logits (launch_paged_logits).
struct SelectArgs {
  const uint16_t* q = nullptr;        // [R,4,128] fp16
  const float* weights = nullptr;     // [R,4] per-head weights, or NULL (all 1)
  const uint16_t* kcache = nullptr;   // [P,128,1,128] fp16 keys, or
  const uint8_t* kcodes = nullptr;    // [P,128,1,128] e4m3 codes, with
  const float* kscale = nullptr;      // [P,128] per-key scales (non-NULL selects e4m3)
  const float* logits_in = nullptr;   // [R, >=logits_width] scores (top-k per row)
  float* logits_out = nullptr;        // [R, logits_width] scores written (paged logits)
  int64_t logits_stride = 0, logits_width = 0;
  int64_t max_visible = 0;            // visible blocks are clamped to this
  const int32_t* block_table = nullptr;  // [N, >=W], row stride bt_stride
  const int32_t* token_to_req = nullptr;
  const int32_t* seq_lens = nullptr;
  const int64_t* query_pos = nullptr;
  int32_t* out = nullptr;             // [R,2051]
  void* workspace = nullptr;
  int64_t rows = 0, num_pages = 0, num_reqs = 0, table_width = 0, bt_stride = 0;
};

// The decode step's selection handed to the attention kernel (the fused
// path): instead of a merge launch, every attention workgroup of a
// multi-chunk row selects the row's top-k from the chunk kernel's
// candidates itself, and the row's last split writes the index row.
struct FusedSelect {
  const uint32_t* cand_keys = nullptr;    // the chunk kernel's candidates
  const uint32_t* cand_blocks = nullptr;
  const int32_t* token_to_req = nullptr;
  const int32_t* seq_lens = nullptr;
  const int64_t* query_pos = nullptr;
  int64_t num_reqs = 0, max_visible = 0, chunks_per_row = 0;
  int chunk_blocks = 0, cand_cap = 0;
};

// A row's candidates the fused path holds in LDS (16 chunks of 512), and
// the merge kernel's batch: plan_select keeps a row within it where the
// largest chunk allows.
constexpr int kFusedCands = 8192;

// A logits row of at most this many columns is selected by one workgroup of
// kRowTopkThreads holding the whole row in LDS (128 KiB of keys).
constexpr int64_t kRowTopkMaxWidth = 32768;
constexpr int kRowTopkThreads = 1024;

struct AttnArgs {
  const uint16_t* q;       // [R,3,256] fp16
  const uint16_t* kv;      // packed rows of 512 fp16 (K at +0, V at +256)
  const int32_t* indices;  // [R,2051] (written for multi-chunk rows when fused)
  const FusedSelect* fused = nullptr;  // non-NULL: select inside the attention
  uint16_t* out;           // [R,3,256] fp16
  void* workspace;
  int64_t rows, num_tokens;
  float scale_log2;        // softmax scale * log2(e)
};

// Arguments of the metadata builder (all device pointers; outputs written).
struct MetaArgs {
  const int32_t* query_start_loc = nullptr;  // [N+1]
  const int32_t* seq_lens = nullptr;         // [N]
  const int32_t* block_table = nullptr;      // [N, table_width], row stride bt_stride
  const int64_t* common_slot_mapping = nullptr;  // [num_tokens] or NULL
  int32_t* token_to_req = nullptr;           // [num_tokens]
  int64_t* logical_positions = nullptr;      // [num_tokens]
  int32_t* visible_blocks = nullptr;         // [num_tokens]
  int64_t* slot_mapping = nullptr;           // [num_tokens] or NULL
  int32_t* k_work = nullptr;                 // [max_num_work][2] or NULL
  int32_t* work_ends = nullptr;              // workspace [N] (with k_work)
  int64_t num_reqs = 0, num_tokens = 0, max_num_work = 0;
  int64_t table_width = 0, bt_stride = 0;
  int64_t storage_block_size = 1, compress_ratio = 1, circular_buffer_size = 0;
};

// Enqueue the kernels; return the hipError_t of the launch (0 = success).
// merge false: launch the chunk kernel only (the fused decode step, whose
// attention kernel does the merge's work).
int launch_select(const SelectArgs& a, const SelectPlan& p, void* stream, bool merge = true);
int launch_paged_logits(const SelectArgs& a, const SelectPlan& p, void* stream);
// Top-k per row over logits rows of at most kRowTopkMaxWidth columns: one
// workgroup of kRowTopkThreads per row, no workspace.
int launch_topk_rows(const SelectArgs& a, void* stream);
int launch_metadata(const MetaArgs& a, void* stream);
int launch_attn(const AttnArgs& a, const AttnPlan& p, void* stream);

// Device address of the calling thread's current device's fixed scratch
// (kStaticScratchBytes, 256-byte aligned); looked up once per device.
// Returns the hipError_t (0 = success).
int static_scratch(void** ptr);

}  // namespace qsa
