// qsa_attn.hip -- fp16 sparse decode attention over [R,2051] logical token
// indices with holes and duplicates, for gfx950.
//
// Implements the attention contract of the page "vLLM: integrate FP16 packed
// QSA extension" ("Exact contracts", attention): Q/output [R,3,256] fp16, a
// packed K/V cache whose token rows hold K in elements 0..255 and V in
// 256..511, index rows of 2051 int32 with -1 holes and repeated entries.
// Every valid position is one softmax member (a repeated index weighs once
// per repetition); a row without valid positions yields zeros.
//
// Design (MI355X / CDNA4): split-K over index positions.
//  * Workgroup (row, split) = 4 waves; each wave walks tiles of 16 index
//    positions.  Per tile, S^T = K_tile . Q^T runs on
//    v_mfma_f32_16x16x32_f16 (A = 16 gathered K rows, lane l loading row
//    l % 16 at bytes [64c + 16(l/16), +16) for c = 0..7; B = the 3 query
//    heads, columns 3..15 zero).  Lane (h + 16g) then holds the logits of
//    head h for positions 4g..4g+3.
//  * Online softmax in base 2 (scale * log2 e folded into the logits), with
//    running max and sum per head, fp32.
//  * P.V on the vector ALU: lane l owns output dims 4l..4l+3 of all three
//    heads; each gathered V row is one coalesced 512-byte wave load; the
//    probabilities are broadcast from the MFMA lanes with v_readlane.
//  * The 4 waves merge in LDS; each workgroup writes its unnormalised
//    partial (max, sum, o[3][256]); a combine kernel merges the splits of a
//    row and rounds to fp16.  With a single split the workgroup writes the
//    final output itself.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_device.h"
#include "qsa_launch.h"
#include "qsa_topk.h"

namespace qsa {
namespace {

constexpr int kThreads = kAttnThreads;  // the split kernel's 4 waves, and the combine's threads
static_assert(kCombineThreads == kAttnThreads, "the combine kernel's thread e owns dim e");

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct AttnParams {
  const uint16_t* q;
  const uint16_t* kv;
  int32_t* indices;  // read; written for multi-chunk rows by the fused path
  uint16_t* out;
  float* partial;  // [rows][splits][3][256]
  float* stats;    // [rows][splits][3][2]
  int64_t rows, num_tokens;
  float scale_log2;
  int splits;
  int split_positions;
  Placement place;  // of the attention (rows x splits) and combine (rows x heads) grids
  FusedSelect sel;  // the fused path's selection inputs
};

template <int kWaves>
struct AttnPart {
  float o[kWaves][kAttHeads][kAttDim];
  float m[kWaves][kAttHeads];
  float l[kWaves][kAttHeads];
};

// The selection prologue's LDS (the merge kernel's work for one row).
template <int NT>
struct SelPart {
  uint32_t keys[kFusedCands];
  uint32_t blocks[kFusedCands];
  uint64_t sorted[kTopKBlocks];
  alignas(16) uint32_t hist0[kBins];
  alignas(16) uint32_t hist1[kBins];
  uint32_t red_and[NT / 64], red_or[NT / 64];
  Scratch s;
};

template <int kWaves, bool kSelect>
struct Smem {
  AttnPart<kWaves> att;
  __device__ AttnPart<kWaves>& part() { return att; }
};

template <int kWaves>
struct Smem<kWaves, true> {
  union {
    AttnPart<kWaves> att;
    SelPart<64 * kWaves> sel;
  } u;
  int32_t idx[kOutWidth + 1];  // the row's selected index list
  __device__ AttnPart<kWaves>& part() { return u.att; }
};

// The index row of a multi-chunk row, selected from the chunk kernel's
// candidates exactly as the merge kernel selects it: the top
// min(512, V) (score descending, block ascending) of the chunks' best keys,
// expanded to tokens with the tail and -1 padding, into idx (LDS).  The
// candidates' shared leading key bits are shifted out before the radix
// select (same order, same ties).  All NT threads call; ends with a barrier.
template <int NT>
__device__ void select_row(const FusedSelect& f, int64_t r, const Row& row, SelPart<NT>& sm,
                           int32_t* idx) {
  const int tid = threadIdx.x;
  const int last_n = (int)(row.visible - (row.nchunks - 1) * f.chunk_blocks);
  const int m = (int)((row.nchunks - 1) * f.cand_cap) + min(f.cand_cap, last_n);
  const int k = (int)min((int64_t)kTopKBlocks, row.visible);
  const uint32_t* ckeys = f.cand_keys + r * f.chunks_per_row * f.cand_cap;
  const uint32_t* cblocks = f.cand_blocks + r * f.chunks_per_row * f.cand_cap;
  for (int i = tid; i < kBins; i += NT) sm.hist0[i] = 0;
  // 16-byte loads (a row's list starts 256-byte aligned; cand_cap is a
  // multiple of 4), two in flight per thread, with the AND and OR of the keys
  uint32_t kand = 0xFFFFFFFFu, kor = 0;
  constexpr int kLoadUnroll = 2;
  const int m4 = m >> 2;
  const uint4* k4 = reinterpret_cast<const uint4*>(ckeys);
  const uint4* b4 = reinterpret_cast<const uint4*>(cblocks);
  for (int j0 = tid; j0 < m4; j0 += NT * kLoadUnroll) {
    uint4 kv[kLoadUnroll], bv[kLoadUnroll];
#pragma unroll
    for (int u = 0; u < kLoadUnroll; ++u) {
      const int j = j0 + u * NT;
      if (j < m4) {
        kv[u] = k4[j];
        bv[u] = b4[j];
      }
    }
#pragma unroll
    for (int u = 0; u < kLoadUnroll; ++u) {
      const int j = j0 + u * NT;
      if (j < m4) {
        const uint32_t xs[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
        const uint32_t bs[4] = {bv[u].x, bv[u].y, bv[u].z, bv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.keys[4 * j + e] = xs[e];
          sm.blocks[4 * j + e] = bs[e];
          kand &= xs[e];
          kor |= xs[e];
        }
      }
    }
  }
  for (int i = 4 * m4 + tid; i < m; i += NT) {
    const uint32_t x = ckeys[i];
    sm.keys[i] = x;
    sm.blocks[i] = cblocks[i];
    kand &= x;
    kor |= x;
  }
  const int shift = shared_lead_bits<NT>(kand, kor, sm.red_and, sm.red_or);
  auto lds_key = [&](int i) { return sm.keys[i] << shift; };
  auto block_of = [&](int i) { return sm.blocks[i]; };
  uint32_t T = 0, bcut = 0xFFFFFFFFu;
  if (m > k) {
    for (int i = tid; i < m; i += NT) atomicAdd(&sm.hist0[digit0(lds_key(i))], 1u);
    __syncthreads();
    topk_threshold<NT>(lds_key, block_of, m, k, (uint32_t)row.visible, sm.s, sm.hist0, sm.hist1, T,
                       bcut);
  }
  compact_topk<NT>(
      lds_key, block_of, m, T, bcut,
      [&](uint32_t slot, int i, uint32_t) { sm.sorted[slot] = pack(sm.keys[i], sm.blocks[i]); },
      sm.s);
  sort_expand_write(sm.sorted, k, row.visible, row.tail, idx, sm.sorted);
  __syncthreads();
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// kWaves waves per workgroup: 4 for splits of a row (kAttnThreads), or
// kAttnRowWaves for about one workgroup per CU.  kSelect (the fused decode
// step): a multi-chunk row's index list is first selected here from the
// chunk kernel's candidates (every split of the row computes the same
// list; the row's last split also writes it out as the index row), then
// the split attends over its positions of that list, exactly as over the
// index row.
template <int kWaves, bool kSelect>
__global__ __launch_bounds__(64 * kWaves) void qsa_attn_kernel(AttnParams p) {
  __shared__ Smem<kWaves, kSelect> sm;
  AttnPart<kWaves>& att = sm.part();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const RowCol id = row_col_of_block(blockIdx.x, p.splits, p.place);
  const int64_t r = id.row;
  const int split = (int)id.col;
  if (r >= p.rows) return;

  const int n = lane & 15;  // token row of A / head column of B
  const int g = lane >> 4;

  // Q^T as the B operand: lane holds head n (if < 3), dims 32c + 8g .. +8.
  half8 qb[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    qb[c] = half8{0, 0, 0, 0, 0, 0, 0, 0};
    if (n < kAttHeads) {
      qb[c] = *reinterpret_cast<const half8*>(p.q + (r * kAttHeads + n) * kAttDim + 32 * c + 8 * g);
    }
  }

  const int32_t* idx_row = p.indices + r * kOutWidth;
  if constexpr (kSelect) {
    const Row row = row_extent(p.sel.token_to_req, p.sel.num_reqs, p.sel.seq_lens,
                               p.sel.query_pos, p.sel.max_visible, p.sel.chunk_blocks, r);
    if (row.nchunks > 1) {  // uniform: rows of one chunk were finished by the chunk kernel
      select_row<64 * kWaves>(p.sel, r, row, sm.u.sel, sm.idx);
      if (split == p.splits - 1) {
        for (int i = tid; i < kOutWidth; i += 64 * kWaves) {
          p.indices[r * kOutWidth + i] = sm.idx[i];
        }
      }
      idx_row = sm.idx;
    }
  }

  const int wave_positions = p.split_positions / kWaves;
  const int pos_begin = split * p.split_positions + wave * wave_positions;
  const int pos_end = min(kOutWidth, pos_begin + wave_positions);
  // The wave's indices come 64 at a time, one per lane, the next 64 loaded
  // while the current ones are used: a tile's gathers wait only for their
  // own data.
  auto group_index = [&](int g0) {
    const int gp = g0 + lane;
    return gp < pos_end ? idx_row[gp] : -1;
  };
  int32_t idx_next = group_index(pos_begin);

  int32_t group_idx = -1;
  bool group_valid = false;
  uint64_t group_mask = 0;
  float m_run = -INFINITY;  // running max of head n (base-2 logits)
  float l_run = 0.f;        // this lane's share of the running sum of head n
  float o[kAttHeads][4];
#pragma unroll
  for (int h = 0; h < kAttHeads; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[h][e] = 0.f;

#pragma unroll 1
  for (int tile = pos_begin; tile < pos_end; tile += 16) {
    const int sub = ((tile - pos_begin) >> 4) & 3;  // tile within its group of 64 positions
    if (sub == 0) {
      group_idx = idx_next;
      group_valid = group_idx >= 0 && group_idx < p.num_tokens;
      group_mask = __ballot(group_valid);
      idx_next = group_index(tile + 64);
    }
    // lane l: the token of position tile + l % 16
    const int32_t idx = __builtin_amdgcn_ds_bpermute(4 * (16 * sub + n), group_valid ? group_idx : 0);
    const int64_t tok = idx;
    const uint64_t vmask = (group_mask >> (16 * sub)) & 0xFFFFull;  // bit t: position tile + t is valid

    // K rows of the 16 positions (A operand) and this lane's slice of the
    // 16 V rows, all issued before any math.
    const half8* kp = reinterpret_cast<const half8*>(p.kv + tok * kKvRow) + g;
    half8 ka[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) ka[c] = kp[4 * c];
    half4 vv[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int64_t tt = __builtin_amdgcn_readlane(idx, t);
      vv[t] = *reinterpret_cast<const half4*>(p.kv + tt * kKvRow + kAttDim + 4 * lane);
    }

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[c], qb[c], acc, 0, 0, 0);
    }
    // lane (h + 16g): logits of head h for positions 4g + v
    float s[4];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const bool ok = (vmask >> (4 * g + v)) & 1ull;
      s[v] = ok ? acc[v] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[v]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f;
    float pr[4] = {0.f, 0.f, 0.f, 0.f};
    if (m_new != -INFINITY) {
      alpha = exp2_fast(m_run - m_new);  // 0 when m_run is -inf
#pragma unroll
      for (int v = 0; v < 4; ++v) pr[v] = exp2_fast(s[v] - m_new);
    }
    m_run = m_new;
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));

#pragma unroll
    for (int h = 0; h < kAttHeads; ++h) {
      const float a = readlane_f(alpha, h);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[h][e] *= a;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float vf[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vf[e] = (float)vv[t][e];
#pragma unroll
      for (int h = 0; h < kAttHeads; ++h) {
        const float pw = readlane_f(pr[t & 3], h + 16 * (t >> 2));
#pragma unroll
        for (int e = 0; e < 4; ++e) o[h][e] = fmaf(pw, vf[e], o[h][e]);
      }
    }
  }

  // per-wave partial: reduce the sum over the four lane groups of a head
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (lane < kAttHeads) {
    att.m[wave][lane] = m_run;
    att.l[wave][lane] = l_run;
  }
#pragma unroll
  for (int h = 0; h < kAttHeads; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) att.o[wave][h][4 * lane + e] = o[h][e];
  __syncthreads();

  // merge the waves: thread t owns (head, dim) pairs t, t + 64 kWaves, ...
#pragma unroll
  for (int he = tid; he < kAttHeads * kAttDim; he += 64 * kWaves) {
    const int h = he / kAttDim, e = he % kAttDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, att.m[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2_fast(att.m[w][h] - M);
        L = fmaf(f, att.l[w][h], L);
        O = fmaf(f, att.o[w][h][e], O);
      }
    }
    if (p.splits == 1) {
      const float y = L > 0.f ? O / L : 0.f;
      const _Float16 yh = (_Float16)y;
      p.out[(r * kAttHeads + h) * kAttDim + e] = *reinterpret_cast<const uint16_t*>(&yh);
    } else {
      const int64_t slot = (r * p.splits + split) * kAttHeads + h;
      p.partial[slot * kAttDim + e] = O;
      if (e == 0) {
        p.stats[slot * 2 + 0] = M;
        p.stats[slot * 2 + 1] = L;
      }
    }
  }
}

// One workgroup per (row, head): wave 0 turns the splits' (max, sum) into
// weights 2^(m_s - M) and the total sum; then thread e sums the weighted
// partials of dim e (independent loads, one per split), normalises, rounds.
constexpr int kMaxSplits = kCombineMaxSplits;  // >= every plan's splits (qsa_launch.h)

__global__ __launch_bounds__(kThreads) void qsa_attn_combine_kernel(AttnParams p) {
  __shared__ float weight[kMaxSplits];
  __shared__ float total;
  const RowCol id = row_col_of_block(blockIdx.x, kAttHeads, p.place);
  const int64_t r = id.row;
  const int h = (int)id.col;
  const int tid = threadIdx.x;
  if (r >= p.rows) return;
  // thread e's partials of the first kPre splits load now, beside the
  // weights' loads (one memory round trip instead of two)
  constexpr int kPre = 8;
  const int e = tid;
  const float* part = p.partial + ((r * p.splits) * kAttHeads + h) * kAttDim + e;
  float pre[kPre];
#pragma unroll
  for (int s = 0; s < kPre; ++s) pre[s] = s < p.splits ? part[(int64_t)s * kAttHeads * kAttDim] : 0.f;
  if (tid < 64) {
    const int s = tid;
    float m = -INFINITY, l = 0.f;
    if (s < p.splits) {
      const int64_t slot = (r * p.splits + s) * kAttHeads + h;
      m = p.stats[slot * 2];
      l = p.stats[slot * 2 + 1];
    }
    float M = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float w = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2_fast(m - M);
    float L = w * l;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
    if (s < kMaxSplits) weight[s] = w;
    if (tid == 0) total = L;
  }
  __syncthreads();
  float O = 0.f;
#pragma unroll
  for (int s = 0; s < kPre; ++s) {
    if (s < p.splits) O = fmaf(weight[s], pre[s], O);
  }
#pragma unroll 8
  for (int s = kPre; s < p.splits; ++s) O = fmaf(weight[s], part[(int64_t)s * kAttHeads * kAttDim], O);
  const float L = total;
  const float y = L > 0.f ? O / L : 0.f;
  const _Float16 yh = (_Float16)y;
  p.out[(r * kAttHeads + h) * kAttDim + e] = *reinterpret_cast<const uint16_t*>(&yh);
}

}  // namespace

int launch_attn(const AttnArgs& a, const AttnPlan& plan, void* stream) {
  if (a.rows == 0) return 0;
  AttnParams p;
  p.q = a.q;
  p.kv = a.kv;
  p.indices = const_cast<int32_t*>(a.indices);
  if (a.fused) p.sel = *a.fused;
  p.out = a.out;
  char* ws = static_cast<char*>(a.workspace);
  p.partial = plan.bytes ? reinterpret_cast<float*>(ws + plan.partial_off) : nullptr;
  p.stats = plan.bytes ? reinterpret_cast<float*>(ws + plan.stats_off) : nullptr;
  p.rows = a.rows;
  p.num_tokens = a.num_tokens;
  p.scale_log2 = a.scale_log2;
  p.splits = plan.splits;
  p.split_positions = plan.split_positions;
  p.place = attn_placement(a.rows);
  const dim3 grid((unsigned)grid_blocks(a.rows, plan.splits, p.place));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.waves == kAttnRowWaves && a.fused) {
    hipLaunchKernelGGL((qsa_attn_kernel<kAttnRowWaves, true>), grid, dim3(64 * kAttnRowWaves), 0,
                       s, p);
  } else if (plan.waves == kAttnRowWaves) {
    hipLaunchKernelGGL((qsa_attn_kernel<kAttnRowWaves, false>), grid, dim3(64 * kAttnRowWaves), 0,
                       s, p);
  } else {
    hipLaunchKernelGGL((qsa_attn_kernel<kAttnThreads / 64, false>), grid, dim3(kAttnThreads), 0,
                       s, p);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.splits == 1) return (int)err;
  hipLaunchKernelGGL(qsa_attn_combine_kernel,
                     dim3((unsigned)grid_blocks(a.rows, kAttHeads, p.place)),
                     dim3(kThreads), 0, s, p);
  return (int)hipGetLastError();
}

}  // namespace qsa
