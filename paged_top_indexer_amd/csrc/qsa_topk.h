// qsa_topk.h -- device helpers of the top-512 selection shared by the
// selection kernels (qsa_select.hip) and the attention kernel's selection
// prologue (qsa_attn.hip): a query row's extent, block-wide radix select
// with the exact tie rule, compaction, and the register bitonic sort that
// orders, expands and writes a row's winners.
//
// The order is the contract's (the page "vLLM: integrate FP16 packed QSA
// extension", "Exact contracts"): score descending, block index ascending
// on exact ties.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kBins = 2048;  // radix digit of up to 11 bits

// Small scratch of the block-wide helpers (at most 4 waves per workgroup).
// The radix histograms are passed separately so that each kernel can place
// them next to data that is dead by then.
struct Scratch {
  uint32_t pick[3];  // digit, rank inside the digit, keys in the digit
  uint32_t count;    // slots handed out by compact_topk
};

struct Row {
  int64_t req = -1;
  int64_t visible = 0;  // V
  int tail = 0;         // T
  int64_t nchunks = 1;
};

// Visible blocks V = max(0, min(floor((qp+1)/4), floor(L/4))) and tail
// T = min(qp+1, L) - 4V of query row r, from its request id `req`, query
// position `qpos` and the request's sequence length.  A request id outside
// [0, N) makes the row empty; V never exceeds what the block table can map
// (or, for a logits source, the logits width).
__device__ inline Row row_from(int64_t req, int64_t qpos, int64_t seq_len, int64_t num_reqs,
                               int64_t max_visible, int chunk_blocks) {
  Row row;
  if (req >= 0 && req < num_reqs) {
    row.req = req;
    const int64_t upto = qpos < INT64_MAX ? qpos + 1 : qpos;
    const int64_t a = upto >= 0 ? upto / kRatio : -1;
    const int64_t b = seq_len >= 0 ? seq_len / kRatio : -1;
    int64_t v = max((int64_t)0, min(a, b));
    const int64_t end = min(upto, seq_len);
    row.tail = (int)max((int64_t)0, min((int64_t)(kRatio - 1), end - kRatio * v));
    row.visible = min(v, max_visible);
  }
  row.nchunks = max((int64_t)1, (row.visible + chunk_blocks - 1) / chunk_blocks);
  return row;
}

// seq_lens[req], read at index 0 for a request id outside [0, N) so that
// the load needs no branch (its value is then unused); N >= 1.
__device__ __forceinline__ int64_t seq_len_at(const int32_t* seq_lens, int64_t num_reqs,
                                              int64_t req) {
  return seq_lens[(req >= 0 && req < num_reqs) ? req : 0];
}

// Row r's extent from the selection inputs: the request id and query
// position are independent loads issued together, then the sequence
// length (two dependent memory round trips, not three).
__device__ inline Row row_extent(const int32_t* token_to_req, int64_t num_reqs,
                                 const int32_t* seq_lens, const int64_t* query_pos,
                                 int64_t max_visible, int chunk_blocks, int64_t r) {
  const int64_t req = token_to_req[r];
  const int64_t qpos = query_pos[r];
  const int64_t seq_len = num_reqs > 0 ? seq_len_at(seq_lens, num_reqs, req) : 0;
  return row_from(req, qpos, seq_len, num_reqs, max_visible, chunk_blocks);
}

// Block-wide: how many leading bits every key of a list shares, from each
// thread's AND and OR of the keys it read (red_and, red_or: one LDS word per
// wave).  Keys shifted left by it keep their order and their ties, and a
// list of one row's best keys -- which share their sign and most of their
// exponent -- spreads over the first radix digit instead of landing in a
// few bins whose LDS atomics would serialise.  All NT threads call; ends
// after a barrier.
template <int NT>
__device__ __forceinline__ int shared_lead_bits(uint32_t kand, uint32_t kor, uint32_t* red_and,
                                                uint32_t* red_or) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kand &= (uint32_t)__shfl_xor((int)kand, o, 64);
    kor |= (uint32_t)__shfl_xor((int)kor, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red_and[threadIdx.x >> 6] = kand;
    red_or[threadIdx.x >> 6] = kor;
  }
  __syncthreads();
  uint32_t all_and = 0xFFFFFFFFu, all_or = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    all_and &= red_and[w];
    all_or |= red_or[w];
  }
  const uint32_t differ = all_and ^ all_or;
  return differ ? __builtin_clz(differ) : 0;
}

// Radix digits of a 32-bit key, most significant first: 11, 11 and 10 bits.
__device__ __forceinline__ uint32_t digit0(uint32_t key) { return key >> 21; }

// Count the keys that match `prefix` under `mask` into h by the digit
// (key >> SHIFT) & (NB - 1).
template <int NT, int SHIFT, int NB, typename KeyAt>
__device__ void radix_count(KeyAt key_at, int n, uint32_t mask, uint32_t prefix, uint32_t* h) {
  constexpr int U = 8;  // keys read before any is counted
  for (int i0 = threadIdx.x; i0 < n; i0 += NT * U) {
    uint32_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = i0 + u * NT < n ? key_at(i0 + u * NT) : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * NT < n && (x[u] & mask) == prefix) {
        atomicAdd(&h[(x[u] >> SHIFT) & (NB - 1)], 1u);
      }
    }
  }
}

// Wave 0 only: find the digit of histogram h (NB bins) that holds the
// krem-th largest counted key.  Lane l reads its NB/64 bins (the digits
// [NB - (l+1)NB/64, NB - l NB/64)) as 16-byte vectors, the wave scans the
// lane sums from the top digit down, and the owning lane walks its bins in
// registers.  Writes (digit, rank inside the digit, keys in the digit).
template <int NB>
__device__ void radix_pick(const uint32_t* h, uint32_t krem, Scratch& s) {
  constexpr int kPer = NB / 64;
  const int lane = threadIdx.x & 63;
  const int lo = NB - kPer * (lane + 1);
  uint32_t c[kPer];
  const uint4* hv = reinterpret_cast<const uint4*>(h + lo);
#pragma unroll
  for (int j = 0; j < kPer / 4; ++j) {
    const uint4 x = hv[j];
    c[4 * j] = x.x;
    c[4 * j + 1] = x.y;
    c[4 * j + 2] = x.z;
    c[4 * j + 3] = x.w;
  }
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) local += c[j];
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t excl = incl - local;
  if (excl < krem && krem <= incl) {
    // (the bin is recorded as its offset j, so that no per-bin index stays
    // live across a caller's loop)
    uint32_t acc = excl, before = 0, count = 0;
    int at = 0;
    bool done = false;
#pragma unroll
    for (int j = kPer - 1; j >= 0; --j) {
      if (!done && acc + c[j] >= krem) {
        at = j;
        before = acc;
        count = c[j];
        done = true;
      }
      acc += c[j];
    }
    s.pick[0] = (uint32_t)(lo + at);
    s.pick[1] = krem - before;
    s.pick[2] = count;
  }
}

// Radix select of the k-th largest (1 <= k <= n) of the keys key_at(i),
// i < n.  On entry hist0 holds the histogram of digit0 over
// all n keys and every thread has passed a barrier since; hist1 is a second
// histogram; both have kBins entries, are 16-byte aligned and may be
// overwritten.  Returns T and need_eq such that the top-k are the keys > T
// plus need_eq of the keys == T, and eq_total = how many keys equal T when
// 0 < need_eq (need_eq == eq_total: all of them).
template <int NT, typename KeyAt>
__device__ void radix_select(KeyAt key_at, int n, int k, Scratch& s, uint32_t* hist0,
                             uint32_t* hist1, uint32_t& T, int& need_eq, int& eq_total) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins; i += NT) hist1[i] = 0;
  if (tid < 64) radix_pick<kBins>(hist0, (uint32_t)k, s);
  __syncthreads();
  uint32_t prefix = s.pick[0] << 21;
  uint32_t mask = (uint32_t)(kBins - 1) << 21;
  uint32_t krem = s.pick[1];
  bool whole = s.pick[2] == krem;  // the boundary bin is taken entirely
  if (!whole) {
    radix_count<NT, 10, kBins>(key_at, n, mask, prefix, hist1);
    for (int i = tid; i < 1024; i += NT) hist0[i] = 0;
    __syncthreads();
    if (tid < 64) radix_pick<kBins>(hist1, krem, s);
    __syncthreads();
    prefix |= s.pick[0] << 10;
    mask |= (uint32_t)(kBins - 1) << 10;
    krem = s.pick[1];
    whole = s.pick[2] == krem;
    if (!whole) {
      radix_count<NT, 0, 1024>(key_at, n, mask, prefix, hist0);
      __syncthreads();
      if (tid < 64) radix_pick<1024>(hist0, krem, s);
      __syncthreads();
      T = prefix | s.pick[0];
      need_eq = (int)s.pick[1];
      eq_total = (int)s.pick[2];
      return;
    }
  }
  // every key >= prefix (lower bits free) is in, nothing else
  if (prefix == 0) {
    T = 0;
    need_eq = eq_total = n;  // all keys
  } else {
    T = prefix - 1;
    need_eq = eq_total = 0;
  }
}

// Threshold of the top-k (1 <= k <= n) under the total order (key
// descending, block ascending): the top-k are the entries with key > T and
// the entries with key == T and block < bcut.  Every block id is below
// block_end (at most 2^31).  Preconditions as for radix_select.  When the
// keys equal to T are only partly in, a second radix select over tie keys
// of those entries (block ids are distinct) finds the last block that is
// in.
template <int NT, typename KeyAt, typename BlockAt>
__device__ void topk_threshold(KeyAt key_at, BlockAt block_at, int n, int k, uint32_t block_end,
                               Scratch& s, uint32_t* hist0, uint32_t* hist1, uint32_t& T,
                               uint32_t& bcut) {
  int need_eq = 0, eq_total = 0;
  radix_select<NT>(key_at, n, k, s, hist0, hist1, T, need_eq, eq_total);
  if (need_eq == 0) {
    bcut = 0;
  } else if (need_eq == eq_total) {
    bcut = 0xFFFFFFFFu;
  } else {
    // Tie key of an entry equal to T: (M - block) << sh with M = 2^B the
    // smallest power of two above every block id -- nonzero, larger for a
    // smaller block, and with the block's significant bits at the top of
    // the word, so that the radix digits resolve them in one pass (B <= 10)
    // or two (B <= 21) rather than spending the first on bits every block
    // shares.  Every other entry's tie key is 0.
    const int B = block_end > 1 ? 32 - __builtin_clz(block_end - 1) : 0;
    const uint32_t M = 1u << B;
    const int sh = 31 - B;
    const uint32_t t = T;
    auto tie_key = [&](int i) { return key_at(i) == t ? (M - block_at(i)) << sh : 0u; };
    for (int i = threadIdx.x; i < kBins; i += NT) hist0[i] = 0;
    __syncthreads();
    // Only the entries equal to T are counted: the others' tie key 0 lies
    // below all of theirs, and need_eq < eq_total of them are taken, so the
    // boundary never falls among the zeros and bin 0 need not hold them
    // (counting them would put nearly every entry's LDS atomic on that one
    // bin).
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t tk = tie_key(i);
      if (tk != 0) atomicAdd(&hist0[digit0(tk)], 1u);
    }
    __syncthreads();
    uint32_t t2 = 0;
    int ne2 = 0, et2 = 0;
    radix_select<NT>(tie_key, n, need_eq, s, hist0, hist1, t2, ne2, et2);
    // The tie keys taken are those > t2, plus t2 itself when ne2 > 0 (tie
    // keys are distinct, so ne2 is 0 or 1; t2 is then an entry's own tie
    // key).  (M - b) << sh > t2 exactly when M - b > t2 >> sh, that is when
    // b < M - (t2 >> sh).
    bcut = (M - (t2 >> sh)) + (ne2 > 0 ? 1u : 0u);
  }
}

// Emit the top-k entries -- key > T, or key == T and block < bcut -- in no
// particular order: emit(slot, i, key) with distinct slots 0..k-1.  One
// pass; each wave ranks its taken lanes with a ballot and reserves slots
// with one LDS atomic per batch of groups.  Ends with a barrier.
template <int NT, typename KeyAt, typename BlockAt, typename Emit>
__device__ void compact_topk(KeyAt key_at, BlockAt block_at, int n, uint32_t T, uint32_t bcut,
                             Emit emit, Scratch& s) {
  constexpr int U = 4;  // 64-key groups per wave and batch
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  if (tid == 0) s.count = 0;
  __syncthreads();
  const int wave_base = tid - lane;
  for (int i0 = wave_base; i0 < n; i0 += NT * U) {
    uint32_t x[U];
    bool take[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + lane;
      x[u] = i < n ? key_at(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + lane;
      take[u] = i < n && (x[u] > T || (x[u] == T && block_at(i) < bcut));
    }
    uint64_t m[U];
    uint32_t total = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m[u] = __ballot(take[u]);
      total += (uint32_t)__popcll(m[u]);
    }
    if (total == 0) continue;  // uniform: the whole wave skips
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&s.count, total);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (take[u]) emit(base + (uint32_t)__popcll(m[u] & below), i0 + u * NT + lane, x[u]);
      base += (uint32_t)__popcll(m[u]);
    }
  }
  __syncthreads();
}

// 64-bit sort key, larger is better: score key in the high word, the
// complement of the block index in the low word (smaller block wins ties).
__device__ __forceinline__ uint64_t pack(uint32_t key, uint32_t block) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - block);
}

// ---- 512-entry bitonic sort held in registers ------------------------------
// A 256-thread workgroup holds the 512 entries two per lane: thread t holds
// entries 2t (a) and 2t+1 (b).  Stride 1 is a swap inside the thread; stride
// s >= 2 pairs lane t with lane t ^ (s/2): inside a wave that is a DPP move
// (lane xor 1, 2, 8), a ds_swizzle (xor 4, 16) or a bpermute (xor 32); only
// strides 128 and 256 cross waves and go through LDS.

template <int X>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (X == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (X == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (X == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (X == 4 || X == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (X << 10) | 0x1F);  // xor within 32
  } else {
    static_assert(X == 32, "lane xor inside a wave");
    return (uint32_t)__shfl_xor((int)v, X, 64);
  }
}

template <int X>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  const uint32_t lo = xor_lane<X>((uint32_t)v);
  const uint32_t hi = xor_lane<X>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// One compare-exchange stage of the descending bitonic network.  Only the
// holders (threads 0..255, whole waves) compute; every thread meets the
// barriers of the LDS stages.
template <int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_stage(uint64_t& a, uint64_t& b, uint64_t* xchg) {
  const int tid = threadIdx.x;
  const bool holder = tid < kTopKBlocks / 2;
  const bool desc = ((2 * tid) & SIZE) == 0;
  if constexpr (STRIDE == 1) {
    if (!holder) return;
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = desc ? hi : lo;
    b = desc ? lo : hi;
  } else {
    constexpr int X = STRIDE / 2;
    uint64_t oa, ob;
    if constexpr (X >= 64) {
      if (holder) {
        xchg[2 * tid] = a;
        xchg[2 * tid + 1] = b;
      }
      __syncthreads();
      oa = holder ? xchg[(2 * tid) ^ STRIDE] : a;
      ob = holder ? xchg[(2 * tid + 1) ^ STRIDE] : b;
      __syncthreads();
    } else {
      if (!holder) return;
      oa = xor_lane64<X>(a);
      ob = xor_lane64<X>(b);
    }
    if (!holder) return;
    const bool keep_hi = ((tid & X) == 0) == desc;
    a = keep_hi ? (a > oa ? a : oa) : (a > oa ? oa : a);
    b = keep_hi ? (b > ob ? b : ob) : (b > ob ? ob : b);
  }
}

template <int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_merge(uint64_t& a, uint64_t& b, uint64_t* xchg) {
  bitonic_stage<SIZE, STRIDE>(a, b, xchg);
  if constexpr (STRIDE > 1) bitonic_merge<SIZE, STRIDE / 2>(a, b, xchg);
}

template <int SIZE>
__device__ __forceinline__ void bitonic_sort(uint64_t& a, uint64_t& b, uint64_t* xchg) {
  if constexpr (SIZE > 2) bitonic_sort<SIZE / 2>(a, b, xchg);
  bitonic_merge<SIZE, SIZE / 2>(a, b, xchg);
}

// The k (<= 512) selected entries list[0..k) (64-bit keys from pack(), any
// order; missing entries count as 0, which sorts last because every real
// entry has a nonzero low word) are sorted descending; each block is
// expanded to its 4 tokens, the tail appended and the row padded with -1.
// Threads 0..255 hold the entries (any workgroup of at least 256 threads;
// all of them must call); needs a barrier between the writes of `list` and
// the call; `xchg` (512 entries) may be `list` itself.
__device__ void sort_expand_write(const uint64_t* list, int k, int64_t visible, int tail,
                                  int32_t* out_row, uint64_t* xchg) {
  const int tid = threadIdx.x;
  uint64_t a = 2 * tid < k ? list[2 * tid] : 0;  // k <= 512: threads >= 256 hold 0
  uint64_t b = 2 * tid + 1 < k ? list[2 * tid + 1] : 0;
  bitonic_sort<kTopKBlocks>(a, b, xchg);
  // thread t holds ranks 2t and 2t+1: tokens 8t .. 8t+7
  const uint64_t mine[2] = {a, b};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rank = 2 * tid + h;
    if (rank < k) {
      const uint32_t block = 0xFFFFFFFFu - (uint32_t)mine[h];
#pragma unroll
      for (int j = 0; j < kRatio; ++j) out_row[kRatio * rank + j] = (int32_t)(kRatio * block + j);
    }
  }
  const int sel_tokens = kRatio * k;
  for (int i = sel_tokens + tid; i < kOutWidth; i += (int)blockDim.x) {
    out_row[i] = i < sel_tokens + tail ? (int32_t)(kRatio * visible + (i - sel_tokens)) : -1;
  }
}

// The same, as a call: inside the chunk kernel's loop over a group's rows
// an inlined sort would keep its LDS exchange addresses live across the
// loop (register spills).
__device__ __noinline__ void sort_expand_write_call(const uint64_t* list, int k, int64_t visible,
                                                    int tail, int32_t* out_row, uint64_t* xchg) {
  sort_expand_write(list, k, visible, tail, out_row, xchg);
}

}  // namespace
}  // namespace qsa
