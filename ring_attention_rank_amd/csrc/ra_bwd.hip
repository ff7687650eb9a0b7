// Backward of one rank's share for bfloat16 inputs with d_k = 128 on gfx950.
//
// Zero to Frontier, "distributed/context-expert", section "Splitting the
// sequence, and the one layer that objects": the backward pass mirrors the
// forward; each GPU computes, from its own queries, the gradients of every
// key/value block it sees (sent back to the block's owner by a reduce-scatter
// in the all-gather form, as a second circulating block in the ring).  Per
// block, with the log-sum-exp the forward returned:
//
//   p = exp(scale q.k - lse),  dp = dout.v,  ds = p (dp - delta),
//   delta = dout.out,  dq += scale ds k,  dk = scale ds^T q,  dv = p^T dout.
//
// Two kernels, each shaped like the forward step kernel so that every
// accumulator stays in registers and nothing is reduced through atomics:
//
//  * dq kernel: a wave owns 32 query rows (Q and dout in registers) and walks
//    the visible 64-key tiles: S^T = K Q^T and dP^T = V dout^T (K and V rows
//    the A operands), dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T (K read
//    transposed, dS^T packed to bf16 as the B operand straight from the
//    accumulators, as P^T feeds V^T P^T in the forward).
//  * dk/dv kernel: the mirror image.  A wave owns 32 keys (K and V rows in
//    registers) and walks every query head of its key/value head and the
//    64-query tiles that see those keys: S = Q K^T and dP = dout V^T (Q and
//    dout rows the A operands), dS = P (dP - delta), dV^T += dout^T P and
//    dK^T += Q^T dS (dout and Q read transposed).
//
// One wave per SIMD (up to 512 registers); tiles are staged through LDS with
// ordinary loads, in two XOR swizzles per tensor (one for row reads, one for
// the transposing ds_read_b64_tr_b16 reads), both free of bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {
namespace bwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int ROWS = 128;      // rows a workgroup owns (4 waves x 32)
constexpr int TILE = 64;       // rows of a staged tile
constexpr int THREADS = 256;
constexpr int TILE_BYTES = TILE * D * 2;  // 16 KiB
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }

// Physical byte offset of 16-byte chunk c of row r: "row" swizzle for
// ds_read_b128 row reads, "tr" swizzle for the transposing reads.
__device__ __forceinline__ int off_row(int r, int c) { return r * 256 + 16 * (c ^ (r & 15)); }
__device__ __forceinline__ int off_tr(int r, int c) { return r * 256 + 16 * (c ^ (4 * (r & 3))); }

// Per-lane read bases (see the forward kernel): row reads of half kb take row
// sigma(col) + 32 kb, logical chunk 2 ks + h; transposing reads give the
// 32 x 16 operand of d block db and row group t of half kb.
struct Lanes {
  int rd_row, rd_tr, h, col;
  __device__ Lanes(int lane) {
    h = lane >> 5;
    col = lane & 31;
    const int r = sigma(col), x = r & 15;
    rd_row = r * 256 + 16 * (h ^ (x & 1)) + 32 * (x >> 1);  // ^ (32 ks)
    const int g4 = lane >> 4, i = lane & 15;
    const int hh = g4 >> 1, dgrp = g4 & 1, rho = i >> 2, b = (i & 3) >> 1, half = i & 1;
    rd_tr = (8 * hh + rho) * 256 + 64 * rho + 32 * dgrp + 16 * b + 8 * half;  // ^ (64 db)
  }
};

__device__ __forceinline__ bf16x8 row_operand(const uint8_t* tile, const Lanes& L, int kb, int ks) {
  return *(const bf16x8*)(tile + kb * 32 * 256 + (L.rd_row ^ (32 * ks)));
}
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* tile, const Lanes& L, int kb, int t,
                                             int db) {
  const uint8_t* base = tile + kb * 32 * 256 + (L.rd_tr ^ (64 * db)) + t * 16 * 256;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * 256));
  // whole-vector assembly: element-wise __bf16 inserts were mis-lowered
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Stages rows [r0, r0 + 64) of a [n][128] bf16 matrix (zeros past n) into
// one or two swizzled LDS tiles.
__device__ __forceinline__ void stage(const uint16_t* src, int r0, int n, uint8_t* t_row,
                                      uint8_t* t_tr, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + THREADS * i;
    const int r = id >> 4, c = id & 15;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r0 + r < n) x = *(const u32x4*)(src + (size_t)(r0 + r) * D + c * 8);
    if (t_row) *(u32x4*)(t_row + off_row(r, c)) = x;
    if (t_tr) *(u32x4*)(t_tr + off_tr(r, c)) = x;
  }
}

// Register value r of half kb of an S^T or S accumulator belongs to tile row
// 32 kb + 8 h + 16 (r / 8) + r % 8.
__device__ __forceinline__ int acc_row(int kb, int h, int r) {
  return 32 * kb + 8 * h + 16 * (r >> 3) + (r & 7);
}

__device__ __forceinline__ void pack(const f32x16& x, bf16x8 (&p)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) p[t][e] = (__bf16)x[8 * t + e];
}

// Stores a 128-wide accumulator (O^T layout: 4 d blocks, lane column = row)
// to row `row` of an fp32 [.][128] matrix, times `mul`, adding the old value
// when ADD.
template <bool ADD>
__device__ __forceinline__ void store_rows(float* dst, const f32x16 (&acc)[4], int h, float mul) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g + e] * mul;
      float* p = dst + db * 32 + 8 * g + 4 * h;
      if (ADD) x += *(const f32x4*)p;
      *(f32x4*)p = x;
    }
}

struct SmemQ {
  uint8_t k_row[TILE_BYTES];
  uint8_t k_tr[TILE_BYTES];
  uint8_t v_row[TILE_BYTES];
  int32_t pos[TILE];
};

// dq kernel: one workgroup = 128 query rows of one head; grid (n_qt, h_q).
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dq_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) SmemQ sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lanes L(lane);
  const int head = blockIdx.y, kvh = head / (a.h_q / a.h_kv);
  const int n_q = a.n_q, n_k = a.n_k;
  const int row0_wg = blockIdx.x * ROWS, row0 = row0_wg + wave * 32;
  const int row = row0 + L.col;
  const bool rv = row < n_q;
  const size_t srow = (size_t)head * n_q + row;

  // queries and their output gradients in registers (B operands)
  const uint16_t* qb = (const uint16_t*)a.q + ((size_t)head * n_q) * D;
  const uint16_t* gb = (const uint16_t*)a.dout + ((size_t)head * n_q) * D;
  bf16x8 q[8], dout[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    q[ks] = rv ? *(const bf16x8*)(qb + (size_t)row * D + ks * 16 + L.h * 8) : bf16x8{};
    dout[ks] = rv ? *(const bf16x8*)(gb + (size_t)row * D + ks * 16 + L.h * 8) : bf16x8{};
  }
  const float lse2 = rv ? a.lse[srow] * kLog2e : -INFINITY;
  const float delta = rv ? a.delta[srow] : 0.f;
  const int qp = rv ? (a.causal ? a.q_pos[row] : 0x7ffffffe) : (int)0x80000000;
  const int n_kt = (n_k + TILE - 1) / TILE;
  int n_iter = n_kt;
  if (a.causal) {
    const int qmax = a.q_pos[min(row0_wg + ROWS, n_q) - 1];
    int cnt = 0;
    for (int j = lane; j < n_kt; j += 64) cnt += a.k_pos[j * TILE] <= qmax ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    n_iter = __builtin_amdgcn_readfirstlane(cnt);
  }
  const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)kvh * n_k) * D;
  const uint16_t* vbase = (const uint16_t*)a.v + ((size_t)kvh * n_k) * D;
  f32x16 dq[4] = {};

  for (int j = 0; j < n_iter; ++j) {
    __syncthreads();
    stage(kbase, j * TILE, n_k, sm.k_row, sm.k_tr, tid);
    stage(vbase, j * TILE, n_k, sm.v_row, nullptr, tid);
    if (tid < TILE) {
      const int gk = j * TILE + tid;
      sm.pos[tid] = gk < n_k ? (a.causal ? a.k_pos[gk] : (int)0x80000000) : 0x7fffffff;
    }
    __syncthreads();
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(sm.k_row, L, kb, ks), q[ks],
                                                        s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(sm.v_row, L, kb, ks),
                                                         dout[ks], dp[kb], 0, 0, 0);
      }
    }
    bf16x8 ds[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 x;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // rows past n_q and rows that saw no key at all have lse = -inf
        const bool vis = sm.pos[acc_row(kb, L.h, r)] <= qp && lse2 != -INFINITY;
        const float p = vis ? exp2f_(__builtin_fmaf(s[kb][r], a.c2, -lse2)) : 0.f;
        x[r] = p * (dp[kb][r] - delta);
      }
      pack(x, ds[kb]);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(sm.k_tr, L, kb, t, db),
                                                           ds[kb][t], dq[db], 0, 0, 0);
  }
  if (rv) store_rows<true>(a.dq + srow * D, dq, L.h, a.scale);
}

struct SmemKV {
  uint8_t q_row[TILE_BYTES];
  uint8_t q_tr[TILE_BYTES];
  uint8_t g_row[TILE_BYTES];
  uint8_t g_tr[TILE_BYTES];
  int32_t pos[TILE];
  float lse2[TILE];
  float delta[TILE];
};

// dk/dv kernel: one workgroup = 128 keys of one key/value head; grid
// (n_kt128, h_kv).  Walks every query head of the group and the query tiles
// that see these keys.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dkv_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) SmemKV sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lanes L(lane);
  const int kvh = blockIdx.y, grp = a.h_q / a.h_kv;
  const int n_q = a.n_q, n_k = a.n_k;
  const int key0_wg = blockIdx.x * ROWS, key0 = key0_wg + wave * 32;
  const int key = key0 + L.col;
  const bool kv = key < n_k;
  const size_t skey = (size_t)kvh * n_k + key;

  const uint16_t* kb_ = (const uint16_t*)a.k + ((size_t)kvh * n_k) * D;
  const uint16_t* vb_ = (const uint16_t*)a.v + ((size_t)kvh * n_k) * D;
  bf16x8 kr[8], vr[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kr[ks] = kv ? *(const bf16x8*)(kb_ + (size_t)key * D + ks * 16 + L.h * 8) : bf16x8{};
    vr[ks] = kv ? *(const bf16x8*)(vb_ + (size_t)key * D + ks * 16 + L.h * 8) : bf16x8{};
  }
  // this lane's key position; keys past the block see nothing
  const int kp = kv ? (a.causal ? a.k_pos[key] : (int)0x80000000) : 0x7fffffff;
  // query tiles that see any of the workgroup's keys form a suffix
  const int n_qt = (n_q + TILE - 1) / TILE;
  int first = 0;
  if (a.causal) {
    const int kmin = a.k_pos[min(key0_wg, n_k - 1)];
    int cnt = 0;  // tiles whose last query precedes kmin
    for (int t = lane; t < n_qt; t += 64) cnt += a.q_pos[min(t * TILE + TILE, n_q) - 1] < kmin ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    first = __builtin_amdgcn_readfirstlane(cnt);
  }
  f32x16 dk[4] = {}, dv[4] = {};

  for (int hg = 0; hg < grp; ++hg) {
    const int head = kvh * grp + hg;
    const uint16_t* qb = (const uint16_t*)a.q + ((size_t)head * n_q) * D;
    const uint16_t* gb = (const uint16_t*)a.dout + ((size_t)head * n_q) * D;
    for (int t0 = first; t0 < n_qt; ++t0) {
      __syncthreads();
      stage(qb, t0 * TILE, n_q, sm.q_row, sm.q_tr, tid);
      stage(gb, t0 * TILE, n_q, sm.g_row, sm.g_tr, tid);
      if (tid < TILE) {
        const int iq = t0 * TILE + tid;
        const bool ok = iq < n_q;
        const size_t sr = (size_t)head * n_q + iq;
        const float l = ok ? a.lse[sr] : -INFINITY;
        sm.pos[tid] = ok ? (a.causal ? a.q_pos[iq] : 0x7ffffffe) : (int)0x80000000;
        sm.lse2[tid] = l * kLog2e;
        sm.delta[tid] = ok ? a.delta[sr] : 0.f;
      }
      __syncthreads();
      f32x16 s[2], dp[2];
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        s[qb2] = f32x16{};
        dp[qb2] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          s[qb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(sm.q_row, L, qb2, ks),
                                                           kr[ks], s[qb2], 0, 0, 0);
          dp[qb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(sm.g_row, L, qb2, ks),
                                                            vr[ks], dp[qb2], 0, 0, 0);
        }
      }
      bf16x8 pp[2][2], ds[2][2];
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        f32x16 p, x;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = acc_row(qb2, L.h, r);
          const float l2 = sm.lse2[qi];
          const bool vis = kp <= sm.pos[qi] && l2 != -INFINITY;
          p[r] = vis ? exp2f_(__builtin_fmaf(s[qb2][r], a.c2, -l2)) : 0.f;
          x[r] = p[r] * (dp[qb2][r] - sm.delta[qi]);
        }
        pack(p, pp[qb2]);
        pack(x, ds[qb2]);
      }
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(sm.g_tr, L, qb2, t, db),
                                                             pp[qb2][t], dv[db], 0, 0, 0);
            dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(sm.q_tr, L, qb2, t, db),
                                                             ds[qb2][t], dk[db], 0, 0, 0);
          }
    }
  }
  if (kv) {
    store_rows<false>(a.dk + skey * D, dk, L.h, a.scale);
    store_rows<false>(a.dv + skey * D, dv, L.h, 1.f);
  }
}

// delta = rowsum(dout * out) per query head and row.
__global__ __launch_bounds__(256) void delta_kernel(const float* out, const uint16_t* dout,
                                                    float* delta, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const float* o = out + r * D;
  const uint16_t* g = dout + r * D;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = lane * 2 + i;
    acc += o[c] * __uint_as_float((uint32_t)g[c] << 16);
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) delta[r] = acc;
}

}  // namespace bwd

hipError_t launch_backward_delta(const float* out, const void* dout, float* delta, int64_t rows,
                                 hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  hipLaunchKernelGGL(bwd::delta_kernel, grid, block, 0, stream, out, (const uint16_t*)dout, delta,
                     rows);
  return hipGetLastError();
}

// dq kernel when there are queries, dk/dv kernel when there are keys (with no
// queries it writes zeros).
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  if (a.n_q > 0) {
    dim3 grid((unsigned)((a.n_q + bwd::ROWS - 1) / bwd::ROWS), (unsigned)a.h_q);
    hipLaunchKernelGGL(bwd::dq_kernel, grid, dim3(bwd::THREADS), 0, stream, a);
  }
  if (a.n_k > 0) {
    dim3 grid((unsigned)((a.n_k + bwd::ROWS - 1) / bwd::ROWS), (unsigned)a.h_kv);
    hipLaunchKernelGGL(bwd::dkv_kernel, grid, dim3(bwd::THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ra
