// ra_forward_noalloc: the ring forward of ra_forward with its workspace (the
// running state and the two staging slots) in a fixed device array instead
// of caller memory, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: every device the library
// runs on holds its own copy from module load until the process ends.  Its
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, together with the five events that order the staging
// copies against the steps; a call after that allocates nothing.
#include <hip/hip_runtime.h>

#include <functional>
#include <mutex>

#include "../../include/ra.h"
#include "ra_internal.h"

namespace {

constexpr size_t kScratchBytes = RA_NOALLOC_MAX_BYTES;  // per device

// The workspace of ra_forward_noalloc.  In host code this name is only a
// handle for hipGetSymbolAddress: the address to pass to kernels and copies is
// the one that call returns (DeviceScratch::ptr).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;  // this device's copy of scratch
  hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  ra_status status = RA_ERR_HIP;  // of the set-up
};
DeviceScratch g_dev[kMaxDevices];

// Runs once per device, with that device current.
void setup(DeviceScratch& d) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return;
  for (hipEvent_t& e : d.ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence) !=
        hipSuccess)
      return;
  d.ptr = p;
  d.status = RA_OK;
}

}  // namespace

extern "C" ra_status ra_forward_noalloc(const ra_problem* p, int32_t n_cp, const void* q,
                                        const int32_t* q_pos, const void* const* k_blocks,
                                        const void* const* v_blocks,
                                        const int32_t* const* k_pos_blocks, float* out, float* lse,
                                        int64_t* work, int64_t* staged_bytes, void* main_stream,
                                        void* side_stream) {
  // The problem first (host checks only), then its size against the array.
  if (p == nullptr) return RA_ERR_NULL;
  int32_t bm = 0, bn = 0;
  const ra_status st = ra_tile_shape(p, &bm, &bn);
  if (st != RA_OK) return st;
  if (ra::forward_noalloc_bytes(p) > kScratchBytes) return RA_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RA_ERR_HIP;
  DeviceScratch& d = g_dev[dev];
  std::call_once(d.once, setup, std::ref(d));
  if (d.status != RA_OK) return d.status;
  return ra::forward_ring(p, n_cp, q, q_pos, k_blocks, v_blocks, k_pos_blocks, d.ptr,
                          kScratchBytes, out, lse, work, staged_bytes, main_stream, side_stream,
                          nullptr, nullptr, d.ev);
}
