// qsa_probe.hip -- libqsa_probe.so (include/qsa_probe.h): a plain
// streaming-read kernel, the practical HBM read ceiling of the box, measured
// beside the path's own kernels.  Not part of the method and not linked into
// its library; it gives the roofline a second, measured denominator.
//
// Each workgroup streams a contiguous span with nontemporal 16-byte loads
// (each load instruction reads 1 KiB contiguous per wave, eight in flight
// per thread) and folds them into an XOR that is stored only if it equals a
// value no real input produces in practice -- the loads cannot be dropped,
// and nothing but the data is read.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/qsa_probe.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 4096;  // 16 per CU
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void qsa_read_probe_kernel(const u32x4* data,
                                                                       int64_t words,
                                                                       uint32_t* sink) {
  // each workgroup streams one contiguous span, 32 KiB per step (as the
  // selection streams 32 KiB pages)
  constexpr int kUnroll = 8;
  constexpr int64_t kStep = (int64_t)kProbeThreads * kUnroll;
  const int64_t span = (words + kProbeBlocks - 1) / kProbeBlocks;
  const int64_t begin = (int64_t)blockIdx.x * span;
  const int64_t end = begin + span < words ? begin + span : words;
  uint32_t acc = 0;
  for (int64_t i0 = begin + threadIdx.x; i0 < end; i0 += kStep) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kProbeThreads;
      v[u] = i < end ? __builtin_nontemporal_load(data + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" QSA_API int qsa_read_probe(const void* data, size_t bytes, void* sink,
                                      size_t sink_bytes, qsa_stream stream) {
  const uintptr_t d = reinterpret_cast<uintptr_t>(data), k = reinterpret_cast<uintptr_t>(sink);
  if (!data || !sink) return QSA_ERR_NULL;
  if (d % 16 || bytes % 16) return QSA_ERR_LAYOUT;
  if (k % 4 || sink_bytes < 4) return QSA_ERR_WORKSPACE;
  if (k < d + bytes && d < k + 4) return QSA_ERR_ALIAS;
  if (bytes == 0) return QSA_OK;
  hipLaunchKernelGGL(qsa_read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(data),
                     (int64_t)(bytes / 16), static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH;
}
