// qsa_noalloc.hip -- the fixed device scratch behind qsa_decode_step_noalloc,
// the decode step for callers that cannot allocate device memory.
//
// The scratch is one file-scope device array: every GPU the library runs on
// holds its own copy (kStaticScratchBytes) from the first use until the
// process ends.  In host code `scratch` names only a host-side stand-in, so
// its device address is looked up once per device (with that device
// current) and kept; host code passes that address to the kernels and never
// the array's name.  Every call on one GPU shares that GPU's array and finds
// the last call's bytes in it: the decode step's kernels write every
// scratch byte they read earlier in the same call, so nothing needs
// clearing, and two calls that overlap on one GPU (different streams) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qsa_launch.h"

static __device__ __align__(256) unsigned char scratch[qsa::kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch[kMaxDevices] = {};

}  // namespace

namespace qsa {

int static_scratch(void** ptr) {
  *ptr = nullptr;
  int device = -1;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return (int)err;
  if (device < 0 || device >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_scratch_lock);
  if (g_scratch[device] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return (int)err;
    g_scratch[device] = p;
  }
  *ptr = g_scratch[device];
  return 0;
}

}  // namespace qsa
