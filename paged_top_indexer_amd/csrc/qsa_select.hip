// qsa_select.hip -- paged top-512 block selection for gfx950.
//
// Implements the selection contract of the page "vLLM: integrate FP16 packed
// QSA extension" (sections "Summary" and "Exact contracts"): paged
// compressed-key gather, four-head ReLU(q.k) scores, top-512 by (score
// descending, block index ascending), expansion of each block to its 4
// tokens, the tail, -1 padding -- no host sync anywhere.  The visible-block
// rule and the page/slot addressing are those of the vllm qsa_cache.py page
// (_build_qsa_metadata_kernel, compressed_qsa_slot_mapping).
//
// Design (MI355X / CDNA4):
//  * Chunk kernel, grid = rows x chunks.  A chunk is `chunk_pages` cache
//    pages (128 compressed keys of 256 B each per page, one contiguous
//    32 KiB run).  Workgroups whose chunk lies past the row's visible blocks
//    exit at once.
//  * Scoring: each wave scores tiles of 16 keys with
//    v_mfma_f32_16x16x32_f16: A = the 4 query heads (rows 4..15 zero),
//    B = 16 keys.  Lane l loads key (l % 16), bytes [64c + 16(l/16), +16)
//    for c = 0..3, so every load instruction reads 16 keys x 64 contiguous
//    bytes.  The 4 head dots of key n land in lane n, so ReLU + head sum is
//    lane-local.  Scores go to LDS as order-preserving uint32 keys (a score
//    is >= 0, so its IEEE bit pattern with the sign bit cleared orders like
//    the value and maps -0 onto +0).
//  * Chunk top-k: an MSB-first radix select (digits of 11, 11 and 9 bits)
//    over the LDS keys finds the k-th largest key T; keys > T are in, keys
//    equal to T are taken in block order until k are in.  Survivors keep
//    block order.  A row that fits in one chunk is sorted, expanded and
//    written right there (one launch does all the work).
//  * Merge kernel, one 1024-thread workgroup per multi-chunk row: the
//    chunks' candidate lists, concatenated in chunk order, are in block
//    order; they are staged through LDS in batches (the running best 512
//    first, so list order stays block order) and reduced with the same radix
//    select.  The winners are bitonic-sorted on the 64-bit key
//    (score << 32 | ~block), expanded and written.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kChunkThreads = 256;
constexpr int kMergeThreads = 1024;
constexpr int kMaxChunkPages = 32;
constexpr int kMaxChunkBlocks = kMaxChunkPages * kPageSlots;  // 4096
constexpr int kUnroll = 4;        // tiles in flight per wave
constexpr int kBins = 2048;       // radix digit of up to 11 bits
constexpr int kMergeList = 8192 + kTopKBlocks;  // LDS list of the merge

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct SelectParams {
  const uint16_t* q;
  const uint16_t* kcache;
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
};

// Scratch shared by the block-wide helpers.
struct Scratch {
  uint32_t hist[kBins];
  uint32_t wave_sum[16];
  uint32_t pick[2];
};

struct Row {
  int64_t req = -1;
  int64_t visible = 0;  // V
  int tail = 0;         // T
  int64_t nchunks = 1;
};

// Visible blocks V = max(0, min(floor((qp+1)/4), floor(L/4))) and tail
// T = min(qp+1, L) - 4V of query row r.  A request id outside [0, N) makes
// the row empty; V never exceeds what the block table can map.
__device__ Row row_setup(const SelectParams& p, int64_t r) {
  Row row;
  const int64_t req = p.token_to_req[r];
  if (req >= 0 && req < p.num_reqs) {
    row.req = req;
    const int64_t seq_len = p.seq_lens[req];
    const int64_t qpos = p.query_pos[r];
    const int64_t upto = qpos < INT64_MAX ? qpos + 1 : qpos;
    const int64_t a = upto >= 0 ? upto / kRatio : -1;
    const int64_t b = seq_len >= 0 ? seq_len / kRatio : -1;
    int64_t v = max((int64_t)0, min(a, b));
    const int64_t end = min(upto, seq_len);
    row.tail = (int)max((int64_t)0, min((int64_t)(kRatio - 1), end - kRatio * v));
    row.visible = min(v, p.table_width * kPageSlots);
  }
  row.nchunks = max((int64_t)1, (row.visible + p.chunk_blocks - 1) / p.chunk_blocks);
  return row;
}

template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, Scratch& s) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) s.wave_sum[wave] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) add += (w < wave) ? s.wave_sum[w] : 0u;
  __syncthreads();
  return v + add;
}

// Radix select: the k-th largest (1 <= k <= n) of the uint32 keys
// key_at(i), i < n, whose bit 31 is clear.  Returns that key T and how many
// keys equal to T belong to the top-k.
template <int NT, typename KeyAt>
__device__ void radix_threshold(KeyAt key_at, int n, int k, Scratch& s, uint32_t& T,
                                int& need_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 9 : 0);
    const int nb = pass == 2 ? 512 : 2048;
    for (int i = tid; i < nb; i += NT) s.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t x = key_at(i);
      if ((x & mask) == prefix) atomicAdd(&s.hist[(x >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns digits nb-1-t*per .. (descending); the scan counts keys
    // at or above each thread's lowest digit
    const int per = (nb + NT - 1) / NT;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) {
      const int d = nb - 1 - (tid * per + j);
      if (d >= 0) local += s.hist[d];
    }
    const uint32_t incl = block_incl_scan<NT>(local, s);
    uint32_t excl = incl - local;
    if (excl < krem && krem <= incl) {
      for (int j = 0; j < per; ++j) {
        const int d = nb - 1 - (tid * per + j);
        if (d < 0) break;
        const uint32_t c = s.hist[d];
        if (excl + c >= krem) {
          s.pick[0] = (uint32_t)d;
          s.pick[1] = krem - excl;
          break;
        }
        excl += c;
      }
    }
    __syncthreads();
    prefix |= s.pick[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    krem = s.pick[1];
    __syncthreads();
  }
  T = prefix;
  need_eq = (int)krem;
}

// Emit the top-k of key_at(0..n) in list order: keys > T and the first
// need_eq keys == T.  emit(slot, i, key) is called with slots 0..k-1.
template <int NT, typename KeyAt, typename Emit>
__device__ void compact_topk(KeyAt key_at, int n, uint32_t T, int need_eq, Emit emit,
                             Scratch& s) {
  const int tid = threadIdx.x;
  const int per = (n + NT - 1) / NT;
  const int beg = min(n, tid * per), end = min(n, beg + per);
  uint32_t gt = 0, eq = 0;
  for (int i = beg; i < end; ++i) {
    const uint32_t x = key_at(i);
    gt += x > T;
    eq += x == T;
  }
  const uint32_t eq_before = block_incl_scan<NT>(eq, s) - eq;
  const int eq_take = max(0, min((int)eq, need_eq - (int)eq_before));
  const uint32_t mine = gt + (uint32_t)eq_take;
  uint32_t slot = block_incl_scan<NT>(mine, s) - mine;
  int eq_seen = 0;
  for (int i = beg; i < end; ++i) {
    const uint32_t x = key_at(i);
    bool take = x > T;
    if (x == T) take = eq_seen++ < eq_take;
    if (take) emit(slot++, i, x);
  }
}

// 64-bit sort key, larger is better: score key in the high word, the
// complement of the block index in the low word (smaller block wins ties).
__device__ __forceinline__ uint64_t pack(uint32_t key, uint32_t block) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - block);
}

// Sort sorted[0..k) descending (entries k..511 padded with 0, which sorts
// last because every real entry has a nonzero low word), expand each block
// to its 4 tokens, append the tail and pad the row with -1.
template <int NT>
__device__ void finalize_row(uint64_t* sorted, int k, int64_t visible, int tail,
                             int32_t* out_row) {
  const int tid = threadIdx.x;
  for (int i = k + tid; i < kTopKBlocks; i += NT) sorted[i] = 0;
  __syncthreads();
#pragma unroll 1
  for (int size = 2; size <= kTopKBlocks; size <<= 1) {
#pragma unroll 1
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (tid < kTopKBlocks / 2) {
        const int i = 2 * tid - (tid & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t a = sorted[i], b = sorted[j];
        if ((a < b) == desc) {
          sorted[i] = b;
          sorted[j] = a;
        }
      }
      __syncthreads();
    }
  }
  const int sel_tokens = kRatio * k;
  for (int i = tid; i < kOutWidth; i += NT) {
    int32_t v = -1;
    if (i < sel_tokens) {
      const uint32_t block = 0xFFFFFFFFu - (uint32_t)sorted[i >> 2];
      v = (int32_t)(kRatio * block + (i & 3));
    } else if (i < sel_tokens + tail) {
      v = (int32_t)(kRatio * visible + (i - sel_tokens));
    }
    out_row[i] = v;
  }
}

struct ChunkSmem {
  uint32_t keys[kMaxChunkBlocks];
  uint64_t sorted[kTopKBlocks];
  Scratch s;
};

__global__ __launch_bounds__(kChunkThreads) void qsa_select_chunk_kernel(SelectParams p) {
  __shared__ ChunkSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t r = blockIdx.x / p.chunks_per_row;
  const int64_t chunk = blockIdx.x % p.chunks_per_row;
  if (r >= p.rows) return;
  const Row row = row_setup(p, r);
  if (chunk >= row.nchunks) return;
  const int64_t chunk_base = chunk * p.chunk_blocks;
  const int nblk = (int)max((int64_t)0, min((int64_t)p.chunk_blocks, row.visible - chunk_base));

  // ---- scoring (MFMA) ----------------------------------------------------
  const int n = lane & 15;  // key column of B / head row of A
  const int g = lane >> 4;  // 8-element slice of each 32-wide k step
  half8 qa[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qa[c] = half8{0, 0, 0, 0, 0, 0, 0, 0};
    if (n < kSelHeads) {
      qa[c] = *reinterpret_cast<const half8*>(p.q + (r * kSelHeads + n) * kSelDim + 32 * c + 8 * g);
    }
  }
  const int32_t* bt_row = p.block_table + row.req * p.bt_stride;
  const int ntiles = (nblk + 15) >> 4;
  constexpr int kWaves = kChunkThreads / 64;
#pragma unroll 1
  for (int t0 = wave; t0 < ntiles; t0 += kWaves * kUnroll) {
    half8 kb[kUnroll][4];
    bool live[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * kWaves;
      live[u] = 16 * t + n < nblk;
      bool load = false;
      const half8* kp = nullptr;
      if (t < ntiles) {
        const int64_t b0 = chunk_base + 16 * t;  // 16-aligned: one page per tile
        const int64_t page = bt_row[b0 >> 7];
        load = live[u] && page >= 0 && page < p.num_pages;
        const int64_t slot = (b0 & (kPageSlots - 1)) + n;
        kp = reinterpret_cast<const half8*>(p.kcache + (page * kPageSlots + slot) * kSelDim) + g;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kb[u][c] = load ? kp[4 * c] : half8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[c], kb[u][c], acc, 0, 0, 0);
      }
      // lanes 0..15 hold heads 0..3 of key n
      const float sc = fmaxf(acc[0], 0.f) + fmaxf(acc[1], 0.f) + fmaxf(acc[2], 0.f) +
                       fmaxf(acc[3], 0.f);
      const int t = t0 + u * kWaves;
      if (g == 0 && live[u]) sm.keys[16 * t + n] = __float_as_uint(sc) & 0x7FFFFFFFu;
    }
  }
  __syncthreads();

  // ---- chunk top-k ---------------------------------------------------------
  const int k_local = min(kTopKBlocks, nblk);
  uint32_t T = 0;
  int need_eq = nblk;  // T = 0 and every key >= 0: all are taken
  auto lds_key = [&](int i) { return sm.keys[i]; };
  if (nblk > kTopKBlocks) radix_threshold<kChunkThreads>(lds_key, nblk, k_local, sm.s, T, need_eq);

  if (row.nchunks == 1) {
    compact_topk<kChunkThreads>(
        lds_key, nblk, T, need_eq,
        [&](uint32_t slot, int i, uint32_t x) { sm.sorted[slot] = pack(x, (uint32_t)(chunk_base + i)); },
        sm.s);
    finalize_row<kChunkThreads>(sm.sorted, k_local, row.visible, row.tail, p.out + r * kOutWidth);
    return;
  }
  const int64_t cbase = (r * p.chunks_per_row + chunk) * p.cand_cap;
  uint32_t* ckeys = p.cand_keys + cbase;
  uint32_t* cblocks = p.cand_blocks + cbase;
  compact_topk<kChunkThreads>(
      lds_key, nblk, T, need_eq,
      [&](uint32_t slot, int i, uint32_t x) {
        ckeys[slot] = x;
        cblocks[slot] = (uint32_t)(chunk_base + i);
      },
      sm.s);
}

struct MergeSmem {
  uint32_t keys[kMergeList];
  uint32_t blocks[kMergeList];
  uint32_t best_keys[kTopKBlocks];
  uint32_t best_blocks[kTopKBlocks];
  uint64_t sorted[kTopKBlocks];
  Scratch s;
};

__global__ __launch_bounds__(kMergeThreads) void qsa_select_merge_kernel(SelectParams p) {
  __shared__ MergeSmem sm;
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  if (r >= p.rows) return;
  const Row row = row_setup(p, r);
  if (row.nchunks == 1) return;  // finished by the chunk kernel

  // Every chunk but the last holds cand_cap candidates, so the row's list is
  // contiguous and in block order.
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
    // list = [running best (earlier blocks)] + [next batch]
    for (int i = tid; i < best_n; i += kMergeThreads) {
      sm.keys[i] = sm.best_keys[i];
      sm.blocks[i] = sm.best_blocks[i];
    }
    for (int i = tid; i < nb; i += kMergeThreads) {
      sm.keys[best_n + i] = ckeys[base + i];
      sm.blocks[best_n + i] = cblocks[base + i];
    }
    __syncthreads();
    const int n_list = best_n + nb;
    const int kk = min(k, n_list);
    uint32_t T = 0;
    int need_eq = n_list;
    auto lds_key = [&](int i) { return sm.keys[i]; };
    if (n_list > kk) radix_threshold<kMergeThreads>(lds_key, n_list, kk, sm.s, T, need_eq);
    compact_topk<kMergeThreads>(
        lds_key, n_list, T, need_eq,
        [&](uint32_t slot, int i, uint32_t x) {
          sm.best_keys[slot] = x;
          sm.best_blocks[slot] = sm.blocks[i];
        },
        sm.s);
    __syncthreads();
    best_n = kk;
  }
  for (int i = tid; i < best_n; i += kMergeThreads) sm.sorted[i] = pack(sm.best_keys[i], sm.best_blocks[i]);
  finalize_row<kMergeThreads>(sm.sorted, best_n, row.visible, row.tail, p.out + r * kOutWidth);
}

}  // namespace

int launch_select(const SelectArgs& a, const SelectPlan& plan, void* stream) {
  if (a.rows == 0) return 0;
  SelectParams p;
  p.q = a.q;
  p.kcache = a.kcache;
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(qsa_select_chunk_kernel, dim3((unsigned)(a.rows * plan.chunks_per_row)),
                     dim3(kChunkThreads), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.chunks_per_row == 1) return (int)err;
  hipLaunchKernelGGL(qsa_select_merge_kernel, dim3((unsigned)a.rows), dim3(kMergeThreads), 0, s, p);
  return (int)hipGetLastError();
}

}  // namespace qsa
