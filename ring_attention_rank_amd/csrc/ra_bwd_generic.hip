// Backward of one rank's share for the shapes the MFMA backward does not take:
// float32 inputs (d_k 64 or 128) and bfloat16 with d_k = 64.  Same
// arithmetic and semantics as the MFMA kernels (Zero to Frontier,
// "distributed/context-expert", section "Splitting the sequence, and the one
// layer that objects": the backward mirrors the forward, each GPU producing
// the gradients of every key/value block it sees):
//
//   p = exp(scale q.k - lse),  ds = p (dout.v - delta),
//   dq += scale ds k,  dk += scale ds q,  dv += p dout,
//
// all in float32 (p and ds are not rounded).  One wave per query row (dq) or
// per key (dk, dv); the d_k elements of a row are spread over the 64 lanes and
// the two dot products per pair are wave reductions.  Correct, not tuned: the
// tuned path is bfloat16 with d_k = 128.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra.h"
#include "ra_internal.h"

namespace ra {
namespace bwdg {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

__device__ __forceinline__ void wave_sum2(float& a, float& b) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off);
    b += __shfl_xor(b, off);
  }
}

// One wave per (head, query row); 4 waves per block.
template <typename T, int D>
__global__ __launch_bounds__(256) void dq_kernel(const BwdArgs a) {
  constexpr int E = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gid >= (int64_t)a.h_q * a.n_q) return;
  const int head = (int)(gid / a.n_q), row = (int)(gid % a.n_q);
  const int kvh = head / (a.h_q / a.h_kv);
  const size_t srow = (size_t)head * a.n_q + row;
  const float lse = a.lse[srow];
  if (lse == -INFINITY) return;  // the row saw no key: nothing to add
  const float lse2 = lse * kLog2e, delta = a.delta[srow];
  const int qp = a.causal ? a.q_pos[row] : 0;
  const T* q = (const T*)a.q + srow * D;
  const T* g = (const T*)a.dout + srow * D;
  const T* kb = (const T*)a.k + (size_t)kvh * a.n_k * D;
  const T* vb = (const T*)a.v + (size_t)kvh * a.n_k * D;
  float qr[E], gr[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qr[e] = ld(q, lane + 64 * e);
    gr[e] = ld(g, lane + 64 * e);
    acc[e] = 0.f;
  }
  for (int j = 0; j < a.n_k; ++j) {
    if (a.causal && a.k_pos[j] > qp) break;  // positions increase: no later key is visible
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      s += qr[e] * ld(kb, (size_t)j * D + lane + 64 * e);
      dp += gr[e] * ld(vb, (size_t)j * D + lane + 64 * e);
    }
    wave_sum2(s, dp);
    const float p = exp2f(s * a.c2 - lse2);
    const float ds = p * (dp - delta);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += ds * ld(kb, (size_t)j * D + lane + 64 * e);
  }
  float* dq = a.dq + srow * D;
#pragma unroll
  for (int e = 0; e < E; ++e) dq[lane + 64 * e] += a.scale * acc[e];
}

// One wave per (key/value head, key); 4 waves per block.  Walks every query
// head of the group and the query rows that see the key (a suffix).
template <typename T, int D>
__global__ __launch_bounds__(256) void dkv_kernel(const BwdArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gid >= (int64_t)a.h_kv * a.n_k) return;
  const int kvh = (int)(gid / a.n_k), key = (int)(gid % a.n_k);
  const int grp = a.h_q / a.h_kv;
  const size_t skey = (size_t)kvh * a.n_k + key;
  const int kp = a.causal ? a.k_pos[key] : 0;
  const T* k = (const T*)a.k + skey * D;
  const T* v = (const T*)a.v + skey * D;
  float kr[E], vr[E], ak[E], av[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kr[e] = ld(k, lane + 64 * e);
    vr[e] = ld(v, lane + 64 * e);
    ak[e] = 0.f;
    av[e] = 0.f;
  }
  // first query row that sees the key (positions increase)
  int first = 0;
  if (a.causal) {
    int lo = 0, hi = a.n_q;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.q_pos[mid] < kp) lo = mid + 1; else hi = mid;
    }
    first = lo;
  }
  for (int hg = 0; hg < grp; ++hg) {
    const int head = kvh * grp + hg;
    const T* qb = (const T*)a.q + (size_t)head * a.n_q * D;
    const T* gb = (const T*)a.dout + (size_t)head * a.n_q * D;
    for (int i = first; i < a.n_q; ++i) {
      const size_t sr = (size_t)head * a.n_q + i;
      const float lse = a.lse[sr];
      if (lse == -INFINITY) continue;  // a row that saw no key adds nothing
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        s += kr[e] * ld(qb, (size_t)i * D + lane + 64 * e);
        dp += vr[e] * ld(gb, (size_t)i * D + lane + 64 * e);
      }
      wave_sum2(s, dp);
      const float p = exp2f(s * a.c2 - lse * kLog2e);
      const float ds = p * (dp - a.delta[sr]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ak[e] += ds * ld(qb, (size_t)i * D + lane + 64 * e);
        av[e] += p * ld(gb, (size_t)i * D + lane + 64 * e);
      }
    }
  }
  float* dk = a.dk + skey * D;
  float* dv = a.dv + skey * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dk[lane + 64 * e] += a.scale * ak[e];
    dv[lane + 64 * e] += av[e];
  }
}

// delta = rowsum(dout * out), one wave per row-head.
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const float* out, const T* dout, float* delta,
                                                    int64_t rows) {
  constexpr int E = D / 64;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  float acc = 0.f, unused = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc += out[r * D + lane + 64 * e] * ld(dout, r * D + lane + 64 * e);
  wave_sum2(acc, unused);
  if (lane == 0) delta[r] = acc;
}

template <typename T, int D>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  const int64_t rq = (int64_t)a.h_q * a.n_q, rk = (int64_t)a.h_kv * a.n_k;
  if (rq > 0 && a.n_k > 0)
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3((unsigned)((rq + 3) / 4)), dim3(256), 0, stream, a);
  if (rk > 0 && a.n_q > 0)
    hipLaunchKernelGGL((dkv_kernel<T, D>), dim3((unsigned)((rk + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_delta(const float* out, const void* dout, float* delta, int64_t rows,
                        hipStream_t stream) {
  hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     out, (const T*)dout, delta, rows);
  return hipGetLastError();
}

}  // namespace bwdg

hipError_t launch_backward_generic(const BwdArgs& a, int dtype, int d_k, hipStream_t stream) {
  if (dtype == RA_F32)
    return d_k == 64 ? bwdg::launch<float, 64>(a, stream) : bwdg::launch<float, 128>(a, stream);
  return d_k == 64 ? bwdg::launch<uint16_t, 64>(a, stream) : bwdg::launch<uint16_t, 128>(a, stream);
}

hipError_t launch_backward_delta_generic(const float* out, const void* dout, float* delta,
                                         int64_t rows, int dtype, int d_k, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (dtype == RA_F32)
    return d_k == 64 ? bwdg::launch_delta<float, 64>(out, dout, delta, rows, stream)
                     : bwdg::launch_delta<float, 128>(out, dout, delta, rows, stream);
  return d_k == 64 ? bwdg::launch_delta<uint16_t, 64>(out, dout, delta, rows, stream)
                   : bwdg::launch_delta<uint16_t, 128>(out, dout, delta, rows, stream);
}

}  // namespace ra
