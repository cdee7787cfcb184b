// qsa_metadata.hip -- QSA metadata for a batch of query tokens, on the GPU
// with no host synchronisation.
//
// Implements the metadata step of the vllm qsa_cache.py page
// (_build_qsa_metadata_kernel and its torch fallback): from the cumulative
// query starts and the sequence lengths, per token
//   request    the last request whose query starts at or before the token
//              (tokens past the mapped ones are padding: request 0),
//   position   seq_len - query_len + (token - query_start) (-1 for padding),
//   visible    max(0, min(floor((position+1)/ratio), floor(seq_len/ratio))),
//   slot       the compressed-cache slot written by the token that completes
//              a group of `ratio` tokens (block table column
//              (position/ratio) / block_size), or the raw-key ring slot
//              (first block, position mod ring size) for the request's last
//              ring-size tokens, or the main cache's slot when neither applies;
// and per request max(floor(L/ratio) - floor((L-q)/ratio), 1) k work items
// for a non-empty query (the first item also commits the raw suffix), laid
// out request after request as (request, index inside the request).
//
// Design: one kernel over max(tokens, work items) threads.  Request search
// and work-owner search are binary searches over the query starts and the
// cumulative work counts.  With at most 4096 requests both live in LDS and
// every workgroup scans the (small) work counts itself, so one launch does
// everything; larger batches search global memory, and their cumulative
// work counts come from a one-workgroup scan kernel launched first.  Scans
// are DPP wave scans.  The mapped-token count is read on the device.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_launch.h"
#include "qsa_device.h"

namespace qsa {
namespace {

constexpr int kMetaThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kLdsReqs = 4096;

__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
  const int64_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}

// Work items of a request with qlen query tokens and seq tokens in all.
__device__ __forceinline__ uint32_t work_count(const MetaArgs& p, int64_t qlen, int64_t seq) {
  if (qlen <= 0) return 0;
  const int64_t groups = floor_div(seq, p.compress_ratio) - floor_div(seq - qlen, p.compress_ratio);
  return (uint32_t)(groups > 1 ? groups : 1);
}

// Inclusive prefix sum of the work counts into ends[0..N) by one workgroup
// of NT threads; qsl(i) reads the query starts.  Ends with a barrier.
template <int NT, typename Qsl>
__device__ void scan_work(const MetaArgs& p, Qsl qsl, int32_t* ends) {
  __shared__ uint32_t wave_sums[NT / 64];
  __shared__ uint32_t carry;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < p.num_reqs; base += NT) {
    const int64_t r = base + tid;
    const uint32_t c = r < p.num_reqs ? work_count(p, qsl(r + 1) - qsl(r), p.seq_lens[r]) : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (lane == 63) wave_sums[wave] = incl;
    __syncthreads();
    uint32_t before = carry;
    for (int w = 0; w < wave; ++w) before += wave_sums[w];
    if (r < p.num_reqs) ends[r] = (int32_t)(before + incl);
    __syncthreads();
    if (tid == NT - 1) carry = before + incl;
    __syncthreads();
  }
}

// Large batches: work_ends[r] = work items of requests 0..r, in global
// memory for the main kernel.
__global__ __launch_bounds__(kScanThreads) void qsa_metadata_scan_kernel(MetaArgs p) {
  scan_work<kScanThreads>(p, [&](int64_t i) -> int64_t { return p.query_start_loc[i]; },
                          p.work_ends);
}

__global__ __launch_bounds__(kMetaThreads) void qsa_metadata_kernel(MetaArgs p) {
  __shared__ int32_t s_qsl[kLdsReqs + 1];
  __shared__ int32_t s_ends[kLdsReqs];
  const int tid = threadIdx.x;
  const int64_t N = p.num_reqs;
  const bool in_lds = N <= kLdsReqs;
  if (in_lds) {
    for (int64_t i = tid; i <= N; i += kMetaThreads) s_qsl[i] = p.query_start_loc[i];
    __syncthreads();
    if (p.k_work) scan_work<kMetaThreads>(p, [&](int64_t i) -> int64_t { return s_qsl[i]; }, s_ends);
  }
  auto qsl = [&](int64_t i) -> int64_t { return in_lds ? s_qsl[i] : p.query_start_loc[i]; };
  auto ends = [&](int64_t i) -> int64_t { return in_lds ? s_ends[i] : p.work_ends[i]; };
  int64_t top = 1;  // largest power of two <= N
  while (top * 2 <= N) top *= 2;

  const int64_t i = (int64_t)blockIdx.x * kMetaThreads + tid;
  if (i < p.num_tokens) {
    const int64_t t = i;
    const int64_t num_mapped = qsl(N);
    const bool mapped = t < num_mapped;
    int64_t r = 0, lp = -1, seq = 0;
    if (mapped) {
      // last r in [0, N) with qsl[r] <= t
      for (int64_t step = top; step > 0; step >>= 1) {
        if (r + step < N && qsl(r + step) <= t) r += step;
      }
      const int64_t start = qsl(r);
      seq = p.seq_lens[r];
      lp = seq - (qsl(r + 1) - start) + (t - start);
    }
    p.token_to_req[t] = (int32_t)r;
    p.logical_positions[t] = lp;
    int64_t v = floor_div(lp + 1, p.compress_ratio);
    const int64_t cap = floor_div(seq, p.compress_ratio);
    v = v < cap ? v : cap;
    p.visible_blocks[t] = (int32_t)(v > 0 ? v : 0);
    if (p.slot_mapping) {
      int64_t slot = -1;
      if (p.circular_buffer_size > 0) {
        const int64_t ring = p.circular_buffer_size;
        if (mapped && lp >= 0 && t + ring >= qsl(r + 1) && p.table_width > 0) {
          const int64_t phys = p.block_table[r * p.bt_stride];
          if (phys >= 0) slot = phys * ring + lp % ring;
        }
      } else if (p.compress_ratio != 1) {
        const int64_t cp = (lp > 0 ? lp : 0) / p.compress_ratio;
        const int64_t lb = cp / p.storage_block_size;
        if (mapped && lp >= 0 && (lp + 1) % p.compress_ratio == 0 && lb < p.table_width) {
          const int64_t phys = p.block_table[r * p.bt_stride + lb];
          const bool live = !p.common_slot_mapping || p.common_slot_mapping[t] >= 0;
          if (phys >= 0 && live) slot = phys * p.storage_block_size + cp % p.storage_block_size;
        }
      } else {
        slot = p.common_slot_mapping ? p.common_slot_mapping[t] : -1;
      }
      p.slot_mapping[t] = slot;
    }
  }

  if (p.k_work && i < p.max_num_work) {
    const int64_t w = i;
    const int64_t total = ends(N - 1);
    int32_t owner = -1, index = -1;
    if (w < total) {
      // first r with ends[r] > w = the number of requests ending at or before w
      int64_t r = 0;
      for (int64_t step = top; step > 0; step >>= 1) {
        if (r + step <= N && ends(r + step - 1) <= w) r += step;
      }
      owner = (int32_t)r;
      index = (int32_t)(w - (r > 0 ? ends(r - 1) : 0));
    }
    p.k_work[2 * w] = owner;
    p.k_work[2 * w + 1] = index;
  }
}

}  // namespace

int launch_metadata(const MetaArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.k_work && a.max_num_work > 0 && a.num_reqs > kLdsReqs) {
    hipLaunchKernelGGL(qsa_metadata_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return (int)err;
  }
  const int64_t items = a.num_tokens > a.max_num_work ? a.num_tokens : a.max_num_work;
  if (items == 0) return 0;
  const int64_t blocks = (items + kMetaThreads - 1) / kMetaThreads;
  hipLaunchKernelGGL(qsa_metadata_kernel, dim3((unsigned)blocks), dim3(kMetaThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace qsa
