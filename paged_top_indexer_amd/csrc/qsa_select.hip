// qsa_select.hip -- paged top-512 block selection for gfx950.
//
// Implements the selection contract of the page "vLLM: integrate FP16 packed
// QSA extension" (sections "Summary" and "Exact contracts"): paged
// compressed-key gather, four-head ReLU(q.k) scores, top-512 by (score
// descending, block index ascending), expansion of each block to its 4
// tokens, the tail, -1 padding -- no host sync anywhere.  The visible-block
// rule and the page/slot addressing are those of the vllm qsa_cache.py page
// (_build_qsa_metadata_kernel, compressed_qsa_slot_mapping).  The same
// kernels serve the two-pass form of the "[XPU] Enable multiple key kernels
// for sparse attention" page (paged logits with per-head weights, then a
// top-k per row over the logits matrix).
//
// Design (MI355X / CDNA4):
//  * Chunk kernel, grid = row groups x chunks.  A chunk is `chunk_pages`
//    cache pages (128 compressed keys of 256 B each per page, one contiguous
//    32 KiB run).  A group is one query row, or up to 4 consecutive rows
//    when the queries come as runs [B, n, 4, 128] (several positions of one
//    request): the group's rows of one request share one read of the keys.
//    Workgroups whose chunk lies past every row's visible blocks exit at
//    once.
//  * Key caches: fp16 keys (256 B each), or e4m3 codes (128 B each) with one
//    fp32 scale per key.  e4m3 codes are decoded to their exact binary16
//    values by the hardware conversion, so the same fp16 MFMA scores both;
//    the key's scale multiplies the head sum (a scale is >= 0, so
//    scale * sum ReLU(q.k) = sum ReLU(q.(scale k))).
//  * Per-head weights (optional, fp32 per row and head) multiply each
//    head's ReLU term; weighted scores may be negative.
//  * Sources and outputs: the chunk kernel scores keys (fp16 or e4m3) or
//    reads scores from a logits matrix, and either selects (top-k) or
//    writes the scores out as logits (-inf past the visible blocks).
//  * Scoring: keys stream in with coalesced nontemporal buffer loads (one
//    instruction = whole keys, 1 KiB contiguous) several 16-key tiles ahead,
//    and pass through a per-wave LDS tile into the B operand of
//    v_mfma_f32_16x16x32_f16; A = 4 heads of up to 4 rows (A row m = head
//    m % 4 of row m / 4), so the 4 head dots of key n for row j land in
//    lane n + 16j and ReLU + head sum is lane-local.  Scores go to LDS as
//    order-preserving uint32 keys (the sign-magnitude bit pattern turned
//    into an unsigned order, -0 mapped onto +0); for a single row the first
//    radix histogram is counted as the scores arrive, under the memory
//    latency.
//  * Chunk top-k of a single row: an MSB-first radix select (digits of 11,
//    11 and 10 bits) finds the k-th largest key; it stops early once the bin
//    holding the k-th key is taken whole.  When keys equal to that threshold
//    are only partly in, a second radix select over the complemented block
//    index of those keys finds the last block that is in, so the tie rule
//    (smaller block first) is decided explicitly and survivors can be
//    compacted in any order (one pass, wave ballots, one LDS atomic per
//    batch).  The rows of a group are selected one per wave, at the same
//    time (a radix select over keys held in registers, no workgroup
//    barriers).  A row that fits in one chunk is sorted, expanded and
//    written right there (one launch does all the work).
//  * Merge kernel, one workgroup per multi-chunk row: the chunks' candidate
//    lists are staged through LDS in batches (behind the running best 512)
//    and reduced with the same select.  The winners are bitonic-sorted in
//    registers on the 64-bit key (score << 32 | ~block), expanded and
//    written.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_launch.h"
#include "qsa_device.h"
#include "qsa_topk.h"

namespace qsa {
namespace {

// (kChunkThreads = 256, kChunkBigThreads = 512 for 64-page chunks;
// kMergeThreads = 768: 3 waves per SIMD hide part of the merge's LDS
// latency -- all in qsa_launch.h)
constexpr int kMaxChunkPages = 64;  // one page per lane
constexpr int kMaxChunkBlocks = 32 * kPageSlots;  // 4096: 4-wave workgroups
// LDS list of the merge: the running best plus a batch of kFusedCands
// candidates (the plans keep a row within one batch where they can)
constexpr int kMergeList = kFusedCands + kTopKBlocks;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SelectParams {
  const uint16_t* q;
  const float* weights;    // [R,4] per-head weights, or NULL (all 1)
  const uint16_t* kcache;  // fp16 keys, or
  const uint8_t* kcodes;   // e4m3 codes [P,128,1,128] with
  const float* kscale;     // one scale per key [P,128]
  const float* logits_in;  // scores given as a logits matrix (top-k per row)
  float* logits_out;       // scores written out (paged logits)
  int64_t logits_stride, logits_width;
  int64_t max_visible;     // visible blocks are clamped to this
  const int32_t* block_table;
  const int32_t* token_to_req;
  const int32_t* seq_lens;
  const int64_t* query_pos;
  int32_t* out;
  uint32_t* cand_keys;    // [rows][chunks_per_row * cand_cap]
  uint32_t* cand_blocks;  // same shape
  int64_t rows, num_pages, num_reqs, table_width, bt_stride;
  int64_t chunks_per_row;
  int chunk_blocks;
  int cand_cap;
  int group;  // consecutive query rows per chunk workgroup (1..4)
  Placement place;  // of the chunk grid (row groups x chunks)
};

// The visible blocks V, tail T and chunks of query row r
// (row_extent in qsa_topk.h) from the selection's inputs.
__device__ Row row_setup(const SelectParams& p, int64_t r) {
  return row_extent(p.token_to_req, p.num_reqs, p.seq_lens, p.query_pos, p.max_visible,
                    p.chunk_blocks, r);
}

// Order-preserving 32-bit key of a score (any finite value or -inf): larger
// key <=> larger score, and -0 maps onto +0, so equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kChunkWaves = kChunkThreads / 64;
constexpr int kWaveBins = 256;  // 8-bit radix digits of the one-wave select
static_assert(kChunkWaves >= kMaxGroup, "one wave per row of a group");
// chunk size of groups of several rows (max_chunk_pages): a wave holds 16
// keys per lane
constexpr int kGroupChunkBlocks = 8 * kPageSlots;
static_assert(kMaxGroup * kGroupChunkBlocks <= kMaxChunkBlocks, "group scores fit in LDS");

// One wave: emit the best min(k, n) of the n keys keys[0..n) (LDS, n <=
// 64 * kPer) under the total order (key descending, index ascending) as
// emit(slot, i, key) with distinct slots 0..min(k, n)-1.  The keys are held
// in registers (lane l takes indices l, l + 64, ...); an MSB-first radix
// select over digits of up to 8 bits, starting at the highest bit in which
// the keys differ (the scores of a chunk share their sign and leading
// exponent bits, which would put every key in one bin), counts into `hist`
// (this wave's kWaveBins entries of LDS) and stops at the first digit whose
// boundary bin is taken whole; keys equal to a fully resolved threshold are
// taken in index order.  No workgroup barrier: the waves of a workgroup
// select different rows at the same time.
template <int kPer, typename Emit>
__device__ void wave_topk(const uint32_t* keys, int n, int k, uint32_t* hist, Emit emit) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t x[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = 64 * u + lane;
    x[u] = i < n ? keys[i] : 0u;
  }
  // selected: keys > T, plus (when need_eq >= 0) the first need_eq keys == T
  // in index order; need_eq < 0 means every key >= T
  uint32_t T = 0;
  int need_eq = -1;
  if (k < n) {
    // bits in which some keys differ: (OR of all) ^ (AND of all)
    uint32_t all_or = 0, all_and = 0xFFFFFFFFu;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (64 * u + lane < n) {
        all_or |= x[u];
        all_and &= x[u];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      all_or |= (uint32_t)__shfl_xor((int)all_or, m);
      all_and &= (uint32_t)__shfl_xor((int)all_and, m);
    }
    const uint32_t differ = all_or ^ all_and;
    int top = differ ? 31 - __builtin_clz(differ) : -1;  // highest differing bit
    // bits every key shares (all of them when the keys are all equal)
    uint32_t pmask = top < 0 ? 0xFFFFFFFFu : top >= 31 ? 0u : ~((2u << top) - 1u);
    uint32_t prefix = all_and & pmask;
    int krem = k;  // rank of the boundary among the keys matching prefix
    bool whole = false;
#pragma unroll 1
    for (; top >= 0 && !whole; top -= 8) {
      const int shift = max(top - 7, 0);
      const uint32_t dmask = (2u << (top - shift)) - 1u;  // digit of bits top..shift
#pragma unroll
      for (int b = lane; b < kWaveBins; b += 64) hist[b] = 0;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (64 * u + lane < n && (x[u] & pmask) == prefix) {
          atomicAdd(&hist[(x[u] >> shift) & dmask], 1u);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // lane l holds the digits 255 - 4l down to 252 - 4l
      const uint4 h = *reinterpret_cast<const uint4*>(hist + kWaveBins - 4 - 4 * lane);
      const uint32_t local = h.x + h.y + h.z + h.w;
      const uint32_t incl = wave_incl_scan(local);
      const uint32_t excl = incl - local;
      const bool owner = excl < (uint32_t)krem && (uint32_t)krem <= incl;
      uint32_t digit = 0, before = 0, count = 0;
      if (owner) {
        const uint32_t c[4] = {h.w, h.z, h.y, h.x};  // digits 255 - 4l - j
        uint32_t acc = excl;
        bool done = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!done && acc + c[j] >= (uint32_t)krem) {
            digit = (uint32_t)(kWaveBins - 1 - 4 * lane - j);
            before = acc;
            count = c[j];
            done = true;
          }
          acc += c[j];
        }
      }
      const int src = __builtin_ctzll(__ballot(owner));
      digit = __builtin_amdgcn_readlane(digit, src);
      before = __builtin_amdgcn_readlane(before, src);
      count = __builtin_amdgcn_readlane(count, src);
      prefix |= digit << shift;
      pmask |= dmask << shift;
      krem -= (int)before;
      whole = (int)count == krem;
    }
    // all bits resolved and the keys equal to T only partly in (or all
    // keys equal): the first krem of them in index order
    T = prefix;
    need_eq = whole ? -1 : krem;
  }
  int base = 0, eq_left = need_eq;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = 64 * u + lane;
    const bool valid = i < n;
    const bool gt = valid && (need_eq < 0 ? x[u] >= T : x[u] > T);
    const bool eq = valid && need_eq >= 0 && x[u] == T;
    const uint64_t meq = __ballot(eq);
    const bool take = gt || (eq && __popcll(meq & below) < eq_left);
    if (need_eq >= 0) eq_left -= min(eq_left, __popcll(meq));
    const uint64_t mt = __ballot(take);
    if (take) emit(base + __popcll(mt & below), i, x[u]);
    base += __popcll(mt);
  }
}

// LDS of a chunk workgroup of kWaves waves over chunks of up to kBlocks
// blocks: 40 KiB for 4 waves and 4096 blocks (four workgroups per CU),
// 72 KiB for 8 waves and 8192 blocks (two).
template <int kWaves, int kBlocks>
struct ChunkSmem {
  static constexpr int kNumWaves = kWaves;
  uint32_t keys[kBlocks];
  alignas(16) uint32_t hist0[kBins];  // counted while scoring
  union {
    // scoring: one 16-key tile per wave, 16-byte chunk j of key n stored at
    // [n][j ^ n] (fp16: 16 chunks per key) or [n][j ^ (n & 7)] (e4m3: 8
    // chunks per key), so that both the coalesced write and the
    // MFMA-layout read touch distinct bank groups
    u32x4 stage[kWaves][16][16];
    u32x4 stage8[kWaves][16][8];
    // selection (after scoring)
    struct {
      alignas(16) uint32_t hist1[kBins];
      uint64_t sorted[kTopKBlocks];
      Scratch s;
    } sel;
    // one wave per row (groups of several rows): a radix histogram per wave
    alignas(16) uint32_t wave_hist[kWaves][kWaveBins];
  } u;
};

// Where a chunk's scores go: score i of the group's row j lands at
// keys[j * stride + i].  For a selection: order-preserving keys, plus the
// first radix histogram when a single-row group's chunk needs a select
// (groups of several rows count it row by row after scoring).
struct LdsSink {
  uint32_t* keys;
  uint32_t* hist0;
  int stride;
  bool count;
  __device__ __forceinline__ void operator()(int j, int i, float sc) const {
    const uint32_t key = score_key(sc);
    keys[j * stride + i] = key;
    if (count) atomicAdd(&hist0[digit0(key)], 1u);
  }
};

// For paged logits: the score itself, staged in LDS; the chunk's logits
// go out in one coalesced pass once the chunk is scored (small scattered
// stores in the middle of the key stream slow the stream down).
struct LogitsSink {
  uint32_t* keys;
  int stride;
  __device__ __forceinline__ void operator()(int j, int i, float sc) const {
    keys[j * stride + i] = __float_as_uint(sc);
  }
};

// The query rows scored in one pass over a chunk's keys: rows r0 + j for
// the set bits j of `mask`, all of one request.  nblk[j] = the chunk's
// blocks visible to row r0 + j (0 outside the mask); the pass streams
// nblk_max keys.
struct PassRows {
  int64_t r0;
  uint32_t mask;
  int nblk[kMaxGroup];
  int nblk_max;
};

// a[j] for a lane-varying j, with constant indices only (the array stays
// in registers).
__device__ __forceinline__ int pick_row(const int (&a)[kMaxGroup], int j) {
  return j == 0 ? a[0] : j == 1 ? a[1] : j == 2 ? a[2] : a[3];
}

// The row's per-head weights (all 1 without a weights tensor) and the
// weighted sum of the ReLU'd head dots of one key (acc[h] = head h).
struct HeadWeights {
  float w[kSelHeads];
};

__device__ __forceinline__ HeadWeights head_weights(const SelectParams& p, int64_t r) {
  HeadWeights hw;
  if (p.weights) {
    const float4 v = *reinterpret_cast<const float4*>(p.weights + r * kSelHeads);
    hw.w[0] = v.x;
    hw.w[1] = v.y;
    hw.w[2] = v.z;
    hw.w[3] = v.w;
  } else {
#pragma unroll
    for (int h = 0; h < kSelHeads; ++h) hw.w[h] = 1.f;
  }
  return hw;
}

__device__ __forceinline__ float head_sum(const floatx4& acc, const HeadWeights& hw) {
  float sum = hw.w[0] * fmaxf(acc[0], 0.f);
#pragma unroll
  for (int h = 1; h < kSelHeads; ++h) sum += hw.w[h] * fmaxf(acc[h], 0.f);
  return sum;
}

// Lane i: the block table's entry for the chunk's i-th logical page of
// request req (at most 64 pages, one per lane), or -1 past the table's
// width, or for an invalid request.  It needs only the request id, so it
// is loaded while the row's sequence length is still in flight (and
// checked only where it is used, so that nothing waits for it early).
__device__ __forceinline__ int32_t page_row(const SelectParams& p, int64_t req, int64_t chunk_base,
                                            int lane) {
  const int64_t col = chunk_base / kPageSlots + lane;
  int32_t entry = -1;
  if (req >= 0 && req < p.num_reqs && lane < p.chunk_blocks / kPageSlots &&
      col < p.table_width) {
    entry = p.block_table[req * p.bt_stride + col];
  }
  return entry;
}

// The physical pages of a chunk of nblk blocks, from its page_row: lane i
// holds the page of the chunk's i-th logical page, or 0 where the valid
// mask is clear -- past the chunk, or an entry outside [0, P) (an unmet
// precondition: such a page reads as an all-zero key).  A tile's page is
// then a readlane away, so no load in the scoring loop waits on another
// load.
__device__ __forceinline__ int32_t chunk_pages(const SelectParams& p, int32_t row_pages, int nblk,
                                               int lane, bool* valid) {
  const int npages = (nblk + kPageSlots - 1) / kPageSlots;
  *valid = lane < npages && row_pages >= 0 && row_pages < p.num_pages;
  return *valid ? row_pages : 0;
}

// Key loads go through a buffer resource spanning one cache page: an offset
// at or past the page's size returns zeros without touching memory.  Keys
// past the chunk's end, tiles past the wave's last one and pages outside
// [0, P) all use such an offset, so every load is unconditional
// (straight-line code: each tile waits only for its own loads) and costs no
// traffic when it is not needed.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
constexpr int kNontemporal = 2;           // cache policy: nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
}

// Keys of tile t (16 blocks from 16t) that exist: 0 when t is past the
// chunk's last tile (tt = the clamped tile) or its page is invalid.
__device__ __forceinline__ int tile_keys(int t, int tt, int ntiles, int nblk, uint64_t valid_mask) {
  const int on_page = (int)((valid_mask >> (tt >> 3)) & 1);
  const int in_chunk = t < ntiles ? min(16, nblk - 16 * tt) : 0;
  return in_chunk * on_page;
}

// fp16 keys.  MFMA k step c covers dims [32c, 32c + 32): lane (n + 16g)
// holds dims [32c + 8g, +8) of key n (B) or of A row n = head n % 4 of the
// pass's row n / 4.  The result of key n for row j (its 4 heads) lands in
// lane n + 16j.
template <typename Smem, typename Sink>
__device__ __forceinline__ void score_chunk_f16(const SelectParams& p, Smem& sm,
                                                const PassRows& pr, int32_t row_pages,
                                                const Sink& sink) {
  constexpr int kWaves = Smem::kNumWaves;
  constexpr int kUnroll = 4;  // tiles in flight per wave (4 KiB each)
  constexpr int kPageBytes = kPageSlots * kSelDim * 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;  // key column of B / row of A
  const int g = lane >> 4;  // 8-element slice of each 32-wide k step / row of the result
  const int nblk = pr.nblk_max;
  half8 qa[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qa[c] = half8{0, 0, 0, 0, 0, 0, 0, 0};
    if ((pr.mask >> (n >> 2)) & 1) {
      const int64_t qrow = (pr.r0 + (n >> 2)) * kSelHeads + (n & 3);
      qa[c] = *reinterpret_cast<const half8*>(p.q + qrow * kSelDim + 32 * c + 8 * g);
    }
  }
  const bool out_row = (pr.mask >> g) & 1;
  const HeadWeights hw = head_weights(p, out_row ? pr.r0 + g : pr.r0);
  const int row_nblk = pick_row(pr.nblk, g);  // 0 for lanes of rows outside the pass
  bool page_valid;
  const int32_t pages = chunk_pages(p, row_pages, nblk, lane, &page_valid);
  const uint64_t valid_mask = __ballot(page_valid);
  const int ntiles = (nblk + 15) >> 4;
  if (wave >= ntiles) return;
  u32x4(*stage)[16] = sm.u.stage[wave];
  const int s16 = lane & 15;  // 16-byte chunk of a key this lane loads

  // Coalesced nontemporal loads: instruction c reads keys 4c..4c+3 of a
  // tile (1 KiB contiguous), lane l taking chunk l % 16 of key 4c + l / 16.
  // Keys are read exactly once; nontemporal loads stream page-permuted
  // reads at the linear-read rate.
  u32x4 raw[kUnroll][4];
  auto issue = [&](int u, int t) {
    // keys of tile t that exist (0 past the wave's last tile or on an
    // invalid page); an integer, so that the compiler keeps one code path
    const int tt = min(t, ntiles - 1);
    const int live = tile_keys(t, tt, ntiles, nblk, valid_mask);
    const int32_t page = __builtin_amdgcn_readlane(pages, tt >> 3);  // 8 tiles per page
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.kcache + (int64_t)page * kPageSlots * kSelDim,
                                                kPageBytes);
    const uint32_t off = (uint32_t)((16 * tt) & (kPageSlots - 1)) * (kSelDim * 2) + lane * 16;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool ok = 4 * c + g < live;
      raw[u][c] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off + 1024 * c : kOutOfRange, 0,
                                                       kNontemporal));
    }
  };
  // Rolling pipeline: slot u holds tile t0 + 4u; once it is scored, the slot
  // is refilled with the tile kUnroll slots ahead, so kUnroll tiles stay in
  // flight while the wave computes.  Every slot is scored on every pass (a
  // slot past the last tile holds zeros and stores nothing): a loop without
  // side exits, so each tile waits only for its own loads.
  // (the scheduling barriers keep the slots' loads in slot order, which the
  // per-tile waits rely on)
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    issue(u, wave + u * kWaves);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll 1
  for (int t0 = wave; t0 < ntiles; t0 += kWaves * kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * kWaves;
      // transpose through the wave's LDS tile
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int key = 4 * c + g;
        stage[key][s16 ^ key] = raw[u][c];
      }
      issue(u, t + kWaves * kUnroll);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_wave_barrier();
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // B operand: lane (n + 16g) holds dims [32c + 8g, +8) of key n
        const half8 kb = __builtin_bit_cast(half8, stage[n][(4 * c + g) ^ n]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[c], kb, acc, 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
      // lane n + 16g holds heads 0..3 of key n for the pass's row g
      const float sc = head_sum(acc, hw);
      if (16 * t + n < row_nblk) sink(g, 16 * t + n, sc);
    }
  }
}

// Eight e4m3 codes (the bytes of w0 then w1, in order) as binary16.  Every
// finite e4m3 value is exact in binary16, and gfx950's
// v_cvt_scalef32_pk_f16_fp8 decodes the OCP e4m3 format two codes at a time
// (word select 0: bytes 0,1; 1: bytes 2,3); with scale 1.0 it is the plain
// conversion.  One instruction per two codes: decoding by integer shifts and
// masks took ~6 vector instructions per pair and made the scorer partly
// ALU-bound.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half8 e4m3x8_to_half8(uint32_t w0, uint32_t w1) {
  const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// e4m3 keys.  The dot product does not care in which order the k steps
// visit the 128 dims, so each lane takes 32 contiguous bytes of its key:
// MFMA k step c gives lane (n + 16g) dims [32g + 8c, +8) of key n (B) or of
// A row n (head n % 4 of the pass's row n / 4); results as for fp16 keys.
// Each wave walks whole pages (pages wave, wave + kWaves, ... of the chunk; eight
// 16-key tiles each), so a page's 128 scales are read once per wave as two
// coalesced 256-byte loads (slots l and 64 + l in lane l), one page ahead,
// and a tile takes its keys' scales from them with a lane permute.
template <typename Smem, typename Sink>
__device__ __forceinline__ void score_chunk_e4m3(const SelectParams& p, Smem& sm,
                                                 const PassRows& pr, int32_t row_pages,
                                                 const Sink& sink) {
  constexpr int kWaves = Smem::kNumWaves;
  constexpr int kUnroll = 8;  // tiles in flight per wave (2 KiB each): one page
  constexpr int kPageBytes = kPageSlots * kSelDim;
  constexpr int kScaleBytes = kPageSlots * 4;
  static_assert(kUnroll * 16 == kPageSlots, "a pipeline pass is one page");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int nblk = pr.nblk_max;
  half8 qa[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qa[c] = half8{0, 0, 0, 0, 0, 0, 0, 0};
    if ((pr.mask >> (n >> 2)) & 1) {
      const int64_t qrow = (pr.r0 + (n >> 2)) * kSelHeads + (n & 3);
      qa[c] = *reinterpret_cast<const half8*>(p.q + qrow * kSelDim + 32 * g + 8 * c);
    }
  }
  const bool out_row = (pr.mask >> g) & 1;
  const HeadWeights hw = head_weights(p, out_row ? pr.r0 + g : pr.r0);
  const int row_nblk = pick_row(pr.nblk, g);
  bool page_valid;
  const int32_t pages = chunk_pages(p, row_pages, nblk, lane, &page_valid);
  const uint64_t valid_mask = __ballot(page_valid);
  const int ntiles = (nblk + 15) >> 4;
  const int npages = (nblk + kPageSlots - 1) / kPageSlots;
  // the wave's tiles: k-th = tile k % 8 of the wave's (k / 8)-th page
  const int nk = npages > wave ? kUnroll * ((npages - wave + kWaves - 1) / kWaves) : 0;
  if (nk == 0) return;
  auto tile_of = [&](int k) { return kUnroll * (wave + kWaves * (k / kUnroll)) + k % kUnroll; };
  u32x4(*stage)[8] = sm.u.stage8[wave];
  const int s8 = lane & 7;     // 16-byte chunk of a key this lane loads
  const int k8 = lane >> 3;    // key of the 8-key half tile this lane loads

  // Coalesced nontemporal loads: instruction c reads keys 8c..8c+7 of a
  // tile (1 KiB contiguous), lane l taking chunk l % 8 of key 8c + l / 8.
  u32x4 raw[kUnroll][2];
  auto issue_keys = [&](int u, int k) {
    const int tt = tile_of(min(k, nk - 1));
    const int on_page = (int)((valid_mask >> (tt >> 3)) & 1);
    const int live = k < nk && tt < ntiles ? min(16, nblk - 16 * tt) * on_page : 0;
    const int32_t page = __builtin_amdgcn_readlane(pages, tt >> 3);
    const __amdgpu_buffer_rsrc_t rk = page_rsrc(p.kcodes + (int64_t)page * kPageSlots * kSelDim,
                                                kPageBytes);
    const uint32_t off = (uint32_t)((16 * tt) & (kPageSlots - 1)) * kSelDim + lane * 16;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool ok = 8 * c + k8 < live;
      raw[u][c] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ok ? off + 1024 * c : kOutOfRange, 0,
                                                       kNontemporal));
    }
  };
  // the 128 scales of the page whose first tile is the wave's k-th
  auto issue_scales = [&](float (&dst)[2], int k) {
    const int pg = tile_of(min(k, nk - 1)) >> 3;  // page within the chunk
    const bool ok = k < nk && ((valid_mask >> pg) & 1);
    const int32_t page = __builtin_amdgcn_readlane(pages, pg);
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(p.kscale + (int64_t)page * kPageSlots, kScaleBytes);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      dst[h] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? (uint32_t)(64 * h + lane) * 4
                                                             : kOutOfRange,
                                                      0, kNontemporal));
    }
  };
  // Rolling pipeline, as in the fp16 scorer, one page per pass: slot u holds
  // tile u of the current page and is refilled with tile u of the next one;
  // the next page's scales are loaded with its first tile (the scheduling
  // barriers keep the loads in the order the per-tile waits rely on).
  float scale_cur[2], scale_next[2];
  issue_scales(scale_cur, 0);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    issue_keys(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll 1
  for (int k0 = 0; k0 < nk; k0 += kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = tile_of(k0 + u);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int key = 8 * c + k8;
        stage[key][s8 ^ (key & 7)] = raw[u][c];
      }
      issue_keys(u, k0 + u + kUnroll);
      if (u == 0) issue_scales(scale_next, k0 + kUnroll);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_wave_barrier();
      const u32x4 lo = stage[n][(2 * g) ^ (n & 7)];      // dims [32g, 32g + 16)
      const u32x4 hi = stage[n][(2 * g + 1) ^ (n & 7)];  // dims [32g + 16, 32g + 32)
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[0], e4m3x8_to_half8(lo[0], lo[1]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[1], e4m3x8_to_half8(lo[2], lo[3]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[2], e4m3x8_to_half8(hi[0], hi[1]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[3], e4m3x8_to_half8(hi[2], hi[3]), acc, 0, 0, 0);
      __builtin_amdgcn_wave_barrier();
      const float sum = head_sum(acc, hw);
      // key n of tile u is page slot 16u + n: in lane (16u + n) % 64 of
      // scale_cur[u / 4]
      const float scale = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(4 * (16 * (u % 4) + n),
                                              __builtin_bit_cast(int, scale_cur[u / 4])));
      // one rounding of scale * code-sum
      const float sc = sum * scale;
      if (16 * tt + n < row_nblk) sink(g, 16 * tt + n, sc);
    }
    scale_cur[0] = scale_next[0];
    scale_cur[1] = scale_next[1];
  }
}

// Scores given as a logits matrix: the chunk's nblk columns of row r.
template <int kThreads, typename Sink>
__device__ __forceinline__ void score_chunk_logits(const SelectParams& p, int64_t r,
                                                   int64_t chunk_base, int nblk, const Sink& sink) {
  constexpr int kUnroll = 8;
  const float* src = p.logits_in + r * p.logits_stride + chunk_base;
#pragma unroll 1
  for (int i0 = threadIdx.x; i0 < nblk; i0 += kThreads * kUnroll) {
    float v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kThreads;
      v[u] = i < nblk ? __builtin_nontemporal_load(src + i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kThreads;
      if (i < nblk) sink(0, i, v[u]);
    }
  }
}

enum : int { kSrcF16 = 0, kSrcE4M3 = 1, kSrcLogits = 2 };



// kSrc: where the scores come from; kLogitsOut: write them as a logits row
// (and -inf past the visible blocks) instead of selecting.  Workgroup (g, c)
// scores chunk c of the rows of group g (p.group consecutive rows; kGroup =
// 1 when p.group is 1, else kMaxGroup); rows of the group that share a
// request are scored in one pass over its keys (a group that spans several
// requests takes one pass per request).
//
// Compiled for 4 waves per SIMD (128 VGPRs; the 40 KiB of LDS allow 4
// workgroups per CU), except the e4m3 scorer over groups of rows: 4 rows x
// 4 heads of queries plus a page of codes in flight need ~148 VGPRs, so it
// runs at 3 waves per SIMD rather than spill to scratch.
template <int kSrc, bool kLogitsOut, int kGroup, int kThreads>
__global__ __launch_bounds__(kThreads, (kSrc == kSrcE4M3 && kGroup > 1) ? 3 : 4) void
qsa_select_chunk_kernel(SelectParams p) {
  static_assert(kThreads == kChunkThreads || kThreads == kChunkBigThreads, "chunk workgroups");
  __shared__ ChunkSmem<kThreads / 64, kThreads == kChunkBigThreads ? 2 * kMaxChunkBlocks
                                                                      : kMaxChunkBlocks> sm;
  const int tid = threadIdx.x;
  const int group = kGroup == 1 ? 1 : p.group;
  const RowCol id = row_col_of_block(blockIdx.x, p.chunks_per_row, p.place);
  const int64_t r0 = id.row * group;
  const int64_t chunk = id.col;
  if (r0 >= p.rows) return;
  const int rows_here = kGroup == 1 ? 1 : (int)min((int64_t)group, p.rows - r0);
  const int64_t chunk_base = chunk * p.chunk_blocks;

  // The group's rows (uniform values, constant indices): request, blocks of
  // this chunk, and which rows have work here (a selection's chunk past a
  // row's last one has none; paged logits fill every column).  Their inputs
  // load in two rounds, each all at once: every row's request id and query
  // position (a group past the batch's end re-reads the last row; unused),
  // then the sequence lengths and the first request's block-table entries
  // for this chunk.
  int64_t req[kMaxGroup], qpos[kMaxGroup], seq[kMaxGroup];
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) {
    req[j] = -1;
    qpos[j] = 0;
    seq[j] = 0;
  }
  // (lane j < kGroup loads row r0 + j's values: one vector load per array
  // and round; per-row scalar loads were issued one after another)
  int32_t pages0 = -1;  // page_row of req[0]
  {
    const int lane = tid & 63;
    const int64_t rl = min(r0 + min(lane, kGroup - 1), p.rows - 1);
    const int32_t req_l = p.token_to_req[rl];
    const int64_t qpos_l = p.query_pos[rl];
    const int64_t req_0 = __builtin_amdgcn_readfirstlane(req_l);
    if constexpr (kSrc != kSrcLogits) pages0 = page_row(p, req_0, chunk_base, lane);
    const int32_t seq_l = p.num_reqs > 0 ? seq_len_at(p.seq_lens, p.num_reqs, req_l) : 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      req[j] = __builtin_amdgcn_readlane(req_l, j);
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)qpos_l, j);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)qpos_l >> 32), j);
      qpos[j] = (int64_t)(((uint64_t)hi << 32) | lo);
      seq[j] = __builtin_amdgcn_readlane(seq_l, j);
    }
  }
  int nblk[kMaxGroup];
  uint32_t live = 0;   // rows with work in this chunk
  uint32_t single = 0; // rows whose only chunk this is (finished here)
  Row row0;
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) {
    nblk[j] = 0;
    if (j < kGroup && j < rows_here) {
      const Row row = row_from(req[j], qpos[j], seq[j], p.num_reqs, p.max_visible, p.chunk_blocks);
      if (j == 0) row0 = row;
      req[j] = row.req;  // -1 for a request id outside [0, N)
      nblk[j] = (int)max((int64_t)0, min((int64_t)p.chunk_blocks, row.visible - chunk_base));
      if (kLogitsOut || chunk < row.nchunks) live |= 1u << j;
      if (row.nchunks == 1) single |= 1u << j;
    } else {
      req[j] = -1;
    }
  }
  if (live == 0) return;

  const bool count_hist = !kLogitsOut && kGroup == 1 && nblk[0] > kTopKBlocks;
  if (count_hist) {
    for (int i = tid; i < kBins; i += kThreads) sm.hist0[i] = 0;
    __syncthreads();
  }
  auto score_all = [&](const auto& sink) {
    if constexpr (kSrc == kSrcLogits) {
      score_chunk_logits<kThreads>(p, r0, chunk_base, nblk[0], sink);  // one row per group
      return;
    }
    uint32_t todo = 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (((live >> j) & 1) && nblk[j] > 0) todo |= 1u << j;
    }
#pragma unroll 1
    while (todo != 0) {
      const int lead = __builtin_ctz(todo);
      const int64_t rq = lead == 0 ? req[0] : lead == 1 ? req[1] : lead == 2 ? req[2] : req[3];
      PassRows pr;
      pr.r0 = r0;
      pr.mask = 0;
      pr.nblk_max = 0;
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j) {
        const bool in = j < kGroup && ((todo >> j) & 1) && req[j] == rq;
        pr.nblk[j] = in ? nblk[j] : 0;
        pr.mask |= in ? 1u << j : 0u;
        pr.nblk_max = max(pr.nblk_max, pr.nblk[j]);
      }
      todo &= ~pr.mask;
      // (the first pass is req[0]'s, whose block-table entries are loaded)
      const int32_t row_pages = rq == req[0] ? pages0 : page_row(p, rq, chunk_base, tid & 63);
      if constexpr (kSrc == kSrcE4M3) {
        score_chunk_e4m3(p, sm, pr, row_pages, sink);
      } else {
        score_chunk_f16(p, sm, pr, row_pages, sink);
      }
    }
  };
  if constexpr (kLogitsOut) {
    score_all(LogitsSink{sm.keys, p.chunk_blocks});
  } else {
    score_all(LdsSink{sm.keys, sm.hist0, p.chunk_blocks, count_hist});
  }
  __syncthreads();

  if constexpr (kLogitsOut) {
#pragma unroll 1
    for (int j = 0; j < rows_here; ++j) {
      const int64_t r = r0 + j;
      const Row row = row_setup(p, r);
      const int nb = (int)max((int64_t)0, min((int64_t)p.chunk_blocks, row.visible - chunk_base));
      float* out_row = p.logits_out + r * p.logits_stride;
      const uint32_t* keys = sm.keys + j * p.chunk_blocks;
      for (int i = tid; i < nb; i += kThreads) {
        __builtin_nontemporal_store(__uint_as_float(keys[i]), out_row + chunk_base + i);
      }
      // -inf from the row's end (or the chunk's start) to the chunk's end;
      // the last chunk column also covers the columns past all chunks
      const int64_t lo = max(row.visible, chunk_base);
      const int64_t hi = chunk == p.chunks_per_row - 1
                             ? p.logits_width
                             : min(chunk_base + (int64_t)p.chunk_blocks, p.logits_width);
      for (int64_t b = lo + tid; b < hi; b += kThreads) out_row[b] = -__builtin_inff();
    }
    return;
  }

  // ---- chunk top-k, row by row ---------------------------------------------
  auto row_topk = [&](int j, const Row& row) {
    const int64_t r = r0 + j;
    const int nb = (int)max((int64_t)0, min((int64_t)p.chunk_blocks, row.visible - chunk_base));
    const bool select = nb > kTopKBlocks;
    const uint32_t* keys = sm.keys + j * p.chunk_blocks;
    if (select && !count_hist) {
      for (int i = tid; i < kBins; i += kThreads) sm.hist0[i] = 0;
      __syncthreads();
      for (int i = tid; i < nb; i += kThreads) atomicAdd(&sm.hist0[digit0(keys[i])], 1u);
      __syncthreads();
    }
    const int k_local = min(kTopKBlocks, nb);
    uint32_t T = 0, bcut = 0xFFFFFFFFu;  // every key >= 0: all are taken
    auto lds_key = [&](int i) { return keys[i]; };
    auto block_of = [&](int i) { return (uint32_t)(chunk_base + i); };
    Scratch& s = sm.u.sel.s;
    if (select) {
      topk_threshold<kThreads>(lds_key, block_of, nb, k_local, (uint32_t)(chunk_base + nb), s,
                               sm.hist0, sm.u.sel.hist1, T, bcut);
    }
    if (row.nchunks == 1) {
      uint64_t* sorted = sm.u.sel.sorted;
      compact_topk<kThreads>(
          lds_key, block_of, nb, T, bcut,
          [&](uint32_t slot, int i, uint32_t x) { sorted[slot] = pack(x, block_of(i)); }, s);
      if constexpr (kGroup == 1) {
        sort_expand_write(sorted, k_local, row.visible, row.tail, p.out + r * kOutWidth, sorted);
      } else {
        sort_expand_write_call(sorted, k_local, row.visible, row.tail, p.out + r * kOutWidth,
                               sorted);
      }
    } else {
      const int64_t cbase = (r * p.chunks_per_row + chunk) * p.cand_cap;
      uint32_t* ckeys = p.cand_keys + cbase;
      uint32_t* cblocks = p.cand_blocks + cbase;
      compact_topk<kThreads>(
          lds_key, block_of, nb, T, bcut,
          [&](uint32_t slot, int i, uint32_t x) {
            ckeys[slot] = x;
            cblocks[slot] = block_of(i);
          },
          s);
    }
  };
  if constexpr (kGroup == 1) {
    row_topk(0, row0);
  } else {
    // rows of several chunks: wave j keeps row j's best keys of the chunk,
    // all rows at once
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (wave < rows_here && (((live & ~single) >> wave) & 1)) {
      const int64_t r = r0 + wave;
      const int64_t cbase = (r * p.chunks_per_row + chunk) * p.cand_cap;
      uint32_t* ckeys = p.cand_keys + cbase;
      uint32_t* cblocks = p.cand_blocks + cbase;
      wave_topk<kGroupChunkBlocks / 64>(
          sm.keys + wave * p.chunk_blocks, pick_row(nblk, wave), kTopKBlocks,
          sm.u.wave_hist[wave], [&](int slot, int i, uint32_t x) {
            ckeys[slot] = x;
            cblocks[slot] = (uint32_t)(chunk_base + i);
          });
    }
    // rows finished here (a single chunk) are sorted and written block-wide
#pragma unroll 1
    for (int j = 0; j < rows_here; ++j) {
      if (((live & single) >> j) & 1) {
        __syncthreads();  // the LDS scratch is free again
        row_topk(j, row_setup(p, r0 + j));
      }
    }
  }
}

struct MergeSmem {
  uint32_t keys[kMergeList];
  uint32_t blocks[kMergeList];
  uint32_t best_keys[kTopKBlocks];
  uint32_t best_blocks[kTopKBlocks];
  uint64_t sorted[kTopKBlocks];
  alignas(16) uint32_t hist0[kBins];
  alignas(16) uint32_t hist1[kBins];
  uint32_t red_and[kMergeThreads / 64], red_or[kMergeThreads / 64];
  Scratch s;
};

__global__ __launch_bounds__(kMergeThreads) void qsa_select_merge_kernel(SelectParams p) {
  __shared__ MergeSmem sm;
  const int tid = threadIdx.x;
  // rows by XCD groups: row s % group of the (s / group)-th run of rows on
  // this XCD (where the chunk kernel places its runs so too, a row is merged
  // on the XCD that scored it)
  const int64_t s = blockIdx.x / kXcds;
  const int64_t r = row_on_xcd(blockIdx.x % kXcds, s / p.group) * p.group + s % p.group;
  if (r >= p.rows) return;
  const Row row = row_setup(p, r);
  if (row.nchunks == 1) return;  // finished by the chunk kernel

  // Every chunk but the last holds cand_cap candidates, so the row's list is
  // contiguous.
  const int last_n = (int)(row.visible - (row.nchunks - 1) * p.chunk_blocks);
  const int m = (int)((row.nchunks - 1) * p.cand_cap) + min(p.cand_cap, last_n);
  const int k = (int)min((int64_t)kTopKBlocks, row.visible);
  const uint32_t* ckeys = p.cand_keys + r * p.chunks_per_row * p.cand_cap;
  const uint32_t* cblocks = p.cand_blocks + r * p.chunks_per_row * p.cand_cap;
  constexpr int kBatch = kMergeList - kTopKBlocks;

  int best_n = 0;
#pragma unroll 1
  for (int base = 0; base < m; base += kBatch) {
    const int nb = min(kBatch, m - base);
    for (int i = tid; i < kBins; i += kMergeThreads) sm.hist0[i] = 0;
    __syncthreads();
    // list = [running best] + [next batch], with the AND and OR of its keys:
    // the candidates are the best keys of their chunks and share their
    // leading bits, so the select runs on the keys shifted left past the
    // bits they all share (same order, same ties; without the shift the
    // first radix digit would put them in a few bins, and the histogram's
    // LDS atomics would serialise)
    uint32_t kand = 0xFFFFFFFFu, kor = 0;
    for (int i = tid; i < best_n; i += kMergeThreads) {
      const uint32_t x = sm.best_keys[i];
      sm.keys[i] = x;
      sm.blocks[i] = sm.best_blocks[i];
      kand &= x;
      kor |= x;
    }
    // 16-byte loads, kLoadUnroll of them in flight per thread (the batch
    // start is a multiple of 4 candidates and the workspace is 256-aligned)
    constexpr int kLoadUnroll = 2;
    const int nb4 = nb >> 2;
    const uint4* k4 = reinterpret_cast<const uint4*>(ckeys + base);
    const uint4* b4 = reinterpret_cast<const uint4*>(cblocks + base);
    for (int j0 = tid; j0 < nb4; j0 += kMergeThreads * kLoadUnroll) {
      uint4 kv[kLoadUnroll], bv[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const int j = j0 + u * kMergeThreads;
        if (j < nb4) {
          kv[u] = k4[j];
          bv[u] = b4[j];
        }
      }
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const int j = j0 + u * kMergeThreads;
        if (j < nb4) {
          const int at = best_n + 4 * j;
          const uint32_t xs[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
          const uint32_t bs[4] = {bv[u].x, bv[u].y, bv[u].z, bv[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sm.keys[at + e] = xs[e];
            sm.blocks[at + e] = bs[e];
            kand &= xs[e];
            kor |= xs[e];
          }
        }
      }
    }
    for (int i = 4 * nb4 + tid; i < nb; i += kMergeThreads) {
      const uint32_t x = ckeys[base + i];
      sm.keys[best_n + i] = x;
      sm.blocks[best_n + i] = cblocks[base + i];
      kand &= x;
      kor |= x;
    }
    const int shift = shared_lead_bits<kMergeThreads>(kand, kor, sm.red_and, sm.red_or);
    const int n_list = best_n + nb;
    const int kk = min(k, n_list);
    auto lds_key = [&](int i) { return sm.keys[i] << shift; };
    auto block_of = [&](int i) { return sm.blocks[i]; };
    if (n_list > kk) {
      for (int i = tid; i < n_list; i += kMergeThreads) atomicAdd(&sm.hist0[digit0(lds_key(i))], 1u);
      __syncthreads();
    }
    uint32_t T = 0, bcut = 0xFFFFFFFFu;
    if (n_list > kk) {
      topk_threshold<kMergeThreads>(lds_key, block_of, n_list, kk, (uint32_t)row.visible, sm.s,
                                    sm.hist0, sm.hist1, T, bcut);
    }
    compact_topk<kMergeThreads>(
        lds_key, block_of, n_list, T, bcut,
        [&](uint32_t slot, int i, uint32_t) {
          sm.best_keys[slot] = sm.keys[i];  // the key itself, not its shifted form
          sm.best_blocks[slot] = sm.blocks[i];
        },
        sm.s);
    best_n = kk;
  }
  for (int i = tid; i < best_n; i += kMergeThreads) sm.sorted[i] = pack(sm.best_keys[i], sm.best_blocks[i]);
  __syncthreads();
  sort_expand_write(sm.sorted, best_n, row.visible, row.tail, p.out + r * kOutWidth, sm.sorted);
}

// ---- top-k per row over a logits matrix, one workgroup per row -----------
// A row of at most kRowTopkMaxWidth scores is held whole in LDS, so one
// workgroup takes it from the logits to the written index row: no chunk
// candidates, no merge launch.  The scores become order-preserving keys as
// they load; the keys' shared leading bits are shifted out before the radix
// select (same order, same ties; without it the first digit would put a
// whole row in a few bins and the histogram's LDS atomics would serialise),
// then threshold, compaction, sort and expansion as in the merge kernel.
struct RowSmem {
  uint32_t keys[kRowTopkMaxWidth];
  alignas(16) uint32_t hist0[kBins];
  alignas(16) uint32_t hist1[kBins];
  uint64_t sorted[kTopKBlocks];
  uint32_t red_and[kRowTopkThreads / 64], red_or[kRowTopkThreads / 64];
  Scratch s;
};

__global__ __launch_bounds__(kRowTopkThreads) void qsa_topk_row_kernel(SelectParams p) {
  __shared__ RowSmem sm;
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  if (r >= p.rows) return;
  for (int i = tid; i < kBins; i += kRowTopkThreads) sm.hist0[i] = 0;
  const Row row = row_setup(p, r);
  const int n = (int)row.visible;  // <= logits_width <= kRowTopkMaxWidth
  const int k = min(kTopKBlocks, n);
  const float* src = p.logits_in + r * p.logits_stride;
  // a whole row in flight at once: 32 loads per thread
  constexpr int kUnroll = kRowTopkMaxWidth / kRowTopkThreads;
  uint32_t kand = 0xFFFFFFFFu, kor = 0;
  for (int i0 = tid; i0 < n; i0 += kRowTopkThreads * kUnroll) {
    float v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kRowTopkThreads;
      v[u] = i < n ? __builtin_nontemporal_load(src + i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kRowTopkThreads;
      if (i < n) {
        const uint32_t key = score_key(v[u]);
        sm.keys[i] = key;
        kand &= key;
        kor |= key;
      }
    }
  }
  const int shift = shared_lead_bits<kRowTopkThreads>(kand, kor, sm.red_and, sm.red_or);
  auto lds_key = [&](int i) { return sm.keys[i] << shift; };
  auto block_of = [&](int i) { return (uint32_t)i; };
  uint32_t T = 0, bcut = 0xFFFFFFFFu;  // k == n: every key is taken
  if (n > k) {
    for (int i = tid; i < n; i += kRowTopkThreads) atomicAdd(&sm.hist0[digit0(lds_key(i))], 1u);
    __syncthreads();
    topk_threshold<kRowTopkThreads>(lds_key, block_of, n, k, (uint32_t)n, sm.s, sm.hist0, sm.hist1,
                                    T, bcut);
  }
  compact_topk<kRowTopkThreads>(
      lds_key, block_of, n, T, bcut,
      [&](uint32_t slot, int i, uint32_t) { sm.sorted[slot] = pack(sm.keys[i], (uint32_t)i); },
      sm.s);
  sort_expand_write(sm.sorted, k, row.visible, row.tail, p.out + r * kOutWidth, sm.sorted);
}

}  // namespace

namespace {

SelectParams make_params(const SelectArgs& a, const SelectPlan& plan) {
  SelectParams p;
  p.q = a.q;
  p.weights = a.weights;
  p.kcache = a.kcache;
  p.kcodes = a.kcodes;
  p.kscale = a.kscale;
  p.logits_in = a.logits_in;
  p.logits_out = a.logits_out;
  p.logits_stride = a.logits_stride;
  p.logits_width = a.logits_width;
  p.max_visible = a.max_visible;
  p.block_table = a.block_table;
  p.token_to_req = a.token_to_req;
  p.seq_lens = a.seq_lens;
  p.query_pos = a.query_pos;
  p.out = a.out;
  char* ws = static_cast<char*>(a.workspace);
  p.cand_keys = plan.bytes ? reinterpret_cast<uint32_t*>(ws + plan.keys_off) : nullptr;
  p.cand_blocks = plan.bytes ? reinterpret_cast<uint32_t*>(ws + plan.blocks_off) : nullptr;
  p.rows = a.rows;
  p.num_pages = a.num_pages;
  p.num_reqs = a.num_reqs;
  p.table_width = a.table_width;
  p.bt_stride = a.bt_stride;
  p.chunks_per_row = plan.chunks_per_row;
  p.chunk_blocks = plan.chunk_pages * kPageSlots;
  p.cand_cap = (int)plan.cand_cap;
  p.group = plan.group;
  p.place = chunk_placement((a.rows + plan.group - 1) / plan.group, plan.group);
  return p;
}

// big: the plan's 64-page chunks of 8-wave workgroups (a selection from
// keys, one row per workgroup); otherwise 4 waves.
template <int kSrc, bool kLogitsOut>
void launch_chunks(const SelectParams& p, bool big, hipStream_t s) {
  const int64_t groups = (p.rows + p.group - 1) / p.group;
  const dim3 grid((unsigned)grid_blocks(groups, p.chunks_per_row, p.place));
  if constexpr (kSrc != kSrcLogits) {  // (logits rows are never grouped)
    if (p.group > 1) {
      hipLaunchKernelGGL((qsa_select_chunk_kernel<kSrc, kLogitsOut, kMaxGroup, kChunkThreads>),
                         grid, dim3(kChunkThreads), 0, s, p);
      return;
    }
    if constexpr (!kLogitsOut) {
      if (big) {
        hipLaunchKernelGGL((qsa_select_chunk_kernel<kSrc, false, 1, kChunkBigThreads>), grid,
                           dim3(kChunkBigThreads), 0, s, p);
        return;
      }
    }
  }
  hipLaunchKernelGGL((qsa_select_chunk_kernel<kSrc, kLogitsOut, 1, kChunkThreads>), grid,
                     dim3(kChunkThreads), 0, s, p);
}

}  // namespace

int launch_select(const SelectArgs& a, const SelectPlan& plan, void* stream, bool merge) {
  if (a.rows == 0) return 0;
  const SelectParams p = make_params(a, plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.logits_in) {
    launch_chunks<kSrcLogits, false>(p, false, s);
  } else if (a.kscale) {
    launch_chunks<kSrcE4M3, false>(p, plan.big, s);
  } else {
    launch_chunks<kSrcF16, false>(p, plan.big, s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.chunks_per_row == 1 || !merge) return (int)err;
  const int64_t groups = (a.rows + p.group - 1) / p.group;
  hipLaunchKernelGGL(qsa_select_merge_kernel, dim3((unsigned)(padded_rows(groups) * p.group)),
                     dim3(kMergeThreads), 0, s, p);
  return (int)hipGetLastError();
}

int launch_topk_rows(const SelectArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  const SelectParams p = make_params(a, SelectPlan{});
  hipLaunchKernelGGL(qsa_topk_row_kernel, dim3((unsigned)a.rows), dim3(kRowTopkThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

int launch_paged_logits(const SelectArgs& a, const SelectPlan& plan, void* stream) {
  if (a.rows == 0) return 0;
  const SelectParams p = make_params(a, plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.kscale) {
    launch_chunks<kSrcE4M3, true>(p, false, s);
  } else {
    launch_chunks<kSrcF16, true>(p, false, s);
  }
  return (int)hipGetLastError();
}

}  // namespace qsa
