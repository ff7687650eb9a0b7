// Matrix-pipe calibration: the sustained rate of v_mfma_f32_32x32x16_bf16
// on this device with nothing else running -- no memory traffic, no VALU
// work beyond the loop -- so that a kernel's achieved rate can be read
// against the clock the chip holds under full matrix-pipe load, not only
// against the nominal 2.4 GHz peak.
#include <hip/hip_runtime.h>

#include "../../include/ra.h"
#include "ra_internal.h"

namespace ra {
namespace calib {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave issues 4 * iters MFMAs on four independent accumulators (the
// pipe never waits on a result), then writes one value per workgroup so the
// work is not dead.  Eight waves per workgroup: two per SIMD.
__global__ __launch_bounds__(512) void mfma_stream_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace calib
}  // namespace ra

extern "C" ra_status ra_mfma_ceiling(int32_t n_workgroups, int32_t iters, float* sink,
                                     void* stream) {
  if (n_workgroups < 1 || iters < 1) return RA_ERR_SHAPE;
  if (!sink) return RA_ERR_NULL;
  if (((uintptr_t)sink & 3) != 0) return RA_ERR_ALIGN;
  hipLaunchKernelGGL(ra::calib::mfma_stream_kernel, dim3((unsigned)n_workgroups), dim3(512), 0,
                     (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}
