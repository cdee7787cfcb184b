// qsa_select.hip -- fused paged top-512 block selection for gfx950.
//
// Implements the selection contract of the page "vLLM: integrate FP16 packed
// QSA extension" (sections "Summary" and "Exact contracts"): paged
// compressed-key gather, four-head ReLU(q.k) scores, top-512 by (score
// descending, block index ascending), expansion of each block to its 4
// tokens, the tail, -1 padding -- all in one launch, no host sync.  The
// visible-block rule and the page/slot addressing are those of the vllm
// qsa_cache.py page (_build_qsa_metadata_kernel, compressed_qsa_slot_mapping).
//
// Design (MI355X / CDNA4):
//  * Grid = rows x chunks.  A chunk is `chunk_pages` cache pages (128
//    compressed keys of 256 B each per page, one contiguous 32 KiB run).
//    Workgroups whose chunk lies past the row's visible blocks exit at once.
//  * Scoring: each wave scores tiles of 16 keys with
//    v_mfma_f32_16x16x32_f16: A = the 4 query heads (rows 4..15 zero),
//    B = 16 keys.  Lane l loads key (l % 16), bytes [64c + 16(l/16), +16)
//    for c = 0..3, so every load instruction reads 16 keys x 64 contiguous
//    bytes.  The 4 head dots of key n land in lane n, so ReLU + head sum is
//    lane-local.  Scores go to LDS as order-preserving uint32 keys (the
//    score is >= 0, so its IEEE bit pattern with the sign cleared orders
//    like the value and maps -0 onto +0).
//  * Per-chunk top-k: an 8-bit MSB-first radix select on the LDS keys finds
//    the k-th largest key T; keys > T are in, keys == T are taken in block
//    order until k are in.  Survivors are written in block order.
//  * The last workgroup of a row to finish (self-resetting atomicInc
//    counter, release/acquire fences) merges the row's chunk candidates
//    with the same radix select, bitonic-sorts the 512 winners by the 64-bit
//    key (score << 32 | ~block), expands and writes the row.  A row that
//    fits in one chunk never touches the workspace.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxChunkPages = 16;
constexpr int kMaxChunkBlocks = kMaxChunkPages * kPageSlots;  // 2048
constexpr int kUnroll = 4;  // tiles in flight per wave

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
  uint32_t* counters;
  uint32_t* cand_keys;
  uint32_t* cand_blocks;
  int64_t rows, num_pages, num_reqs, table_width, bt_stride;
  int64_t chunks_per_row;
  int chunk_blocks;
  int cand_cap;
};

struct Smem {
  uint32_t keys[kMaxChunkBlocks];
  uint64_t sorted[kTopKBlocks];
  uint32_t hist[256];
  uint32_t wave_sum[kWaves];
  uint32_t pick[2];
  uint32_t last;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum over the 256 threads of the workgroup.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, Smem& sm) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sm.wave_sum[wave] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) add += (w < wave) ? sm.wave_sum[w] : 0u;
  __syncthreads();
  return v + add;
}

// Radix select: the k-th largest (1 <= k <= n) of the uint32 keys key_at(i),
// i < n.  Returns the key T and how many keys equal to T belong to the top-k.
template <typename KeyAt>
__device__ void radix_threshold(KeyAt key_at, int n, int k, Smem& sm, uint32_t& T,
                                int& need_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)k;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    sm.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      uint32_t x = key_at(i);
      if ((x & mask) == prefix) atomicAdd(&sm.hist[(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t counts digit 255 - t: the scan gives how many keys have a
    // digit >= 255 - t; the digit holding the krem-th largest is found where
    // that count first reaches krem.
    uint32_t c = sm.hist[255 - tid];
    uint32_t incl = block_incl_scan(c, sm);
    uint32_t excl = incl - c;
    if (excl < krem && krem <= incl) {
      sm.pick[0] = 255u - tid;
      sm.pick[1] = krem - excl;
    }
    __syncthreads();
    prefix |= sm.pick[0] << shift;
    mask |= 255u << shift;
    krem = sm.pick[1];
    __syncthreads();
  }
  T = prefix;
  need_eq = (int)krem;
}

// Emit the top-k of key_at(0..n) in list order: keys > T, and the first
// need_eq keys == T.  emit(slot, i, key) is called with slot = 0..k-1.
template <typename KeyAt, typename Emit>
__device__ void compact_topk(KeyAt key_at, int n, uint32_t T, int need_eq, Emit emit,
                             Smem& sm) {
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int beg = min(n, tid * per), end = min(n, beg + per);
  uint32_t gt = 0, eq = 0;
  for (int i = beg; i < end; ++i) {
    uint32_t x = key_at(i);
    gt += x > T;
    eq += x == T;
  }
  const uint32_t eq_before = block_incl_scan(eq, sm) - eq;
  const int eq_take = max(0, min((int)eq, need_eq - (int)eq_before));
  const uint32_t mine = gt + (uint32_t)eq_take;
  uint32_t slot = block_incl_scan(mine, sm) - mine;
  int eq_seen = 0;
  for (int i = beg; i < end; ++i) {
    uint32_t x = key_at(i);
    bool take = x > T;
    if (x == T) take = eq_seen++ < eq_take;
    if (take) emit(slot++, i, x);
  }
}

// 64-bit sort key: larger is better.  Score key in the high word, the
// complement of the block index in the low word (smaller block wins ties).
__device__ __forceinline__ uint64_t pack(uint32_t key, uint32_t block) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - block);
}

// Sort sm.sorted[0..k) descending (entries k..511 padded with 0, which sorts
// last because every real entry has a nonzero low word), expand and write.
__device__ void finalize_row(Smem& sm, int k, int64_t visible, int tail, int32_t* out_row) {
  const int tid = threadIdx.x;
  for (int i = k + tid; i < kTopKBlocks; i += kThreads) sm.sorted[i] = 0;
  __syncthreads();
#pragma unroll 1
  for (int size = 2; size <= kTopKBlocks; size <<= 1) {
#pragma unroll 1
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int i = 2 * tid - (tid & (stride - 1));
      const int j = i + stride;
      const bool desc = (i & size) == 0;
      const uint64_t a = sm.sorted[i], b = sm.sorted[j];
      if ((a < b) == desc) {
        sm.sorted[i] = b;
        sm.sorted[j] = a;
      }
      __syncthreads();
    }
  }
  const int sel_tokens = kRatio * k;
  for (int i = tid; i < kOutWidth; i += kThreads) {
    int32_t v = -1;
    if (i < sel_tokens) {
      const uint32_t block = 0xFFFFFFFFu - (uint32_t)sm.sorted[i >> 2];
      v = (int32_t)(kRatio * block + (i & 3));
    } else if (i < sel_tokens + tail) {
      v = (int32_t)(kRatio * visible + (i - sel_tokens));
    }
    out_row[i] = v;
  }
}

__global__ __launch_bounds__(kThreads) void qsa_select_kernel(SelectParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int64_t r = blockIdx.x / p.chunks_per_row;
  const int64_t chunk = blockIdx.x % p.chunks_per_row;
  if (r >= p.rows) return;

  // ---- row setup: visible blocks V and tail T ----------------------------
  const int64_t req = p.token_to_req[r];
  int64_t visible = 0;
  int tail = 0;
  if (req >= 0 && req < p.num_reqs) {
    const int64_t seq_len = p.seq_lens[req];
    const int64_t qpos = p.query_pos[r];
    const int64_t upto = qpos < INT64_MAX ? qpos + 1 : qpos;
    const int64_t a = upto >= 0 ? upto / kRatio : -1;
    const int64_t b = seq_len >= 0 ? seq_len / kRatio : -1;
    visible = max((int64_t)0, min(a, b));
    const int64_t end = min(upto, seq_len);
    tail = (int)max((int64_t)0, min((int64_t)(kRatio - 1), end - kRatio * visible));
    // never read past the block table (a violated precondition)
    visible = min(visible, p.table_width * kPageSlots);
  }
  const int64_t nchunks = max((int64_t)1, (visible + p.chunk_blocks - 1) / p.chunk_blocks);
  if (chunk >= nchunks) return;
  const int64_t chunk_base = chunk * p.chunk_blocks;
  const int nblk = (int)max((int64_t)0, min((int64_t)p.chunk_blocks, visible - chunk_base));

  // ---- scoring (MFMA) ----------------------------------------------------
  const int n = lane & 15;  // key column of the B operand / head row of A
  const int g = lane >> 4;  // which 8-element slice of each 32-wide k step
  half8 qa[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qa[c] = half8{0, 0, 0, 0, 0, 0, 0, 0};
    if (n < kSelHeads) {
      qa[c] = *reinterpret_cast<const half8*>(p.q + (r * kSelHeads + n) * kSelDim + 32 * c + 8 * g);
    }
  }
  const int32_t* bt_row = p.block_table + req * p.bt_stride;
  const int ntiles = (nblk + 15) >> 4;
#pragma unroll 1
  for (int t0 = wave; t0 < ntiles; t0 += kWaves * kUnroll) {
    half8 kb[kUnroll][4];
    bool live[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * kWaves;
      const int pos = 16 * t + n;  // block offset inside the chunk
      live[u] = pos < nblk;
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
      const float s = fmaxf(acc[0], 0.f) + fmaxf(acc[1], 0.f) + fmaxf(acc[2], 0.f) +
                      fmaxf(acc[3], 0.f);
      const int t = t0 + u * kWaves;
      if (g == 0 && live[u]) sm.keys[16 * t + n] = __float_as_uint(s) & 0x7FFFFFFFu;
    }
  }
  __syncthreads();

  // ---- local top-k ---------------------------------------------------------
  const int k_local = min(kTopKBlocks, nblk);
  uint32_t T = 0;
  int need_eq = 0;
  auto lds_key = [&](int i) { return sm.keys[i]; };
  if (nblk > kTopKBlocks) {
    radix_threshold(lds_key, nblk, k_local, sm, T, need_eq);
  } else {
    need_eq = nblk;  // T = 0 and every key >= 0: all are taken
  }

  int32_t* out_row = p.out + r * kOutWidth;
  if (nchunks == 1) {
    compact_topk(lds_key, nblk, T, need_eq,
                 [&](uint32_t slot, int i, uint32_t x) {
                   sm.sorted[slot] = pack(x, (uint32_t)(chunk_base + i));
                 },
                 sm);
    finalize_row(sm, k_local, visible, tail, out_row);
    return;
  }

  uint32_t* ckeys = p.cand_keys + r * p.chunks_per_row * p.cand_cap;
  uint32_t* cblocks = p.cand_blocks + r * p.chunks_per_row * p.cand_cap;
  const int64_t cbase = chunk * p.cand_cap;
  compact_topk(lds_key, nblk, T, need_eq,
               [&](uint32_t slot, int i, uint32_t x) {
                 ckeys[cbase + slot] = x;
                 cblocks[cbase + slot] = (uint32_t)(chunk_base + i);
               },
               sm);

  // ---- last workgroup of the row merges ------------------------------------
  __threadfence();  // release this workgroup's candidates
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicInc(&p.counters[r], (uint32_t)(nchunks - 1));
    sm.last = prev == (uint32_t)(nchunks - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  __threadfence();  // acquire the other chunks' candidates

  // Non-last chunks are full (cand_cap candidates each), so the row's list
  // is contiguous and in block order.
  const int last_n = (int)min((int64_t)p.chunk_blocks, visible - (nchunks - 1) * p.chunk_blocks);
  const int m = (int)((nchunks - 1) * p.cand_cap) + min(p.cand_cap, last_n);
  const int k = (int)min((int64_t)kTopKBlocks, visible);
  auto gkey = [&](int i) { return __builtin_nontemporal_load(&ckeys[i]); };
  if (m > k) {
    radix_threshold(gkey, m, k, sm, T, need_eq);
  } else {
    T = 0;
    need_eq = m;
  }
  compact_topk(gkey, m, T, need_eq,
               [&](uint32_t slot, int i, uint32_t x) { sm.sorted[slot] = pack(x, cblocks[i]); },
               sm);
  finalize_row(sm, k, visible, tail, out_row);
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
  p.counters = plan.bytes ? reinterpret_cast<uint32_t*>(ws + plan.counters_off) : nullptr;
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
  const int64_t grid = a.rows * plan.chunks_per_row;
  hipLaunchKernelGGL(qsa_select_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace qsa
