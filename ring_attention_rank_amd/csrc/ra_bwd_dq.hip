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
//  * dk/dv kernel (ra_bwd_dkv.hip): the mirror image.  A wave owns 32 keys
//    (K and V rows in registers) and walks the query heads of its split of
//    the key/value head's group and the 64-query tiles that see those keys:
//    S = Q K^T and dP = dout V^T (Q and dout rows the A operands),
//    dS = P (dP - delta), dV^T += dout^T P and dK^T += Q^T dS (dout and Q
//    read transposed).
//
// One wave per SIMD (up to 512 registers).  Each 64-row tile is loaded into
// registers one tile ahead, then written to LDS in two XOR swizzles per
// tensor (one for row reads, one for the transposing ds_read_b64_tr_b16
// reads), both free of bank conflicts.  Inside a tile the instructions are
// fenced in issue order: every MFMA goes out with the LDS operand reads four
// MFMAs ahead and a slice of the other half-tile's VALU work.
//
// This unit: the dq kernel and delta = rowsum(dout * out).  Its MFMA
// accumulators live in ordinary VGPRs (built with the VGPR form), so the
// softmax-gradient VALU work reads them without moves.
#include "ra_bwd_common.h"

namespace ra {
namespace bwd {

// 1024-byte aligned: the second buffer keeps the 16-byte chunk alignment and
// the bank mapping of the swizzles.
struct __attribute__((aligned(1024))) TileQ {
  uint8_t k_row[TILE_BYTES];
  uint8_t k_tr[TILE_BYTES];
  uint8_t v_row[TILE_BYTES];
  int32_t pos[TILE];
};
// Two tile buffers: tile j is read from t[j & 1] while tile j + 1 is written
// into the other one, slice by slice between the MFMAs.
struct SmemQ {
  TileQ t[2];
};

// LDS operand reads run this many MFMAs ahead of their use.
constexpr int AHEAD = 4;

// dq kernel: one workgroup = 128 query rows of one head; a one-dimensional
// grid of n_qt128 * h_q workgroups.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dq_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) SmemQ sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lanes L(lane);
  int bx, head;  // heads that share a key/value head on one XCD
  xcd_split(blockIdx.x, a.h_q, bx, head);
  const int kvh = head / (a.h_q / a.h_kv);
  const int n_q = a.n_q, n_k = a.n_k;
  const int row0_wg = bx * ROWS, row0 = row0_wg + wave * 32;
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
  // q and dout land before any tile load is issued, so the waits inside the
  // tile loop only ever concern the prefetch of the next tile
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  // rows past n_q and rows that saw no key at all have lse = -inf: p = 0
  const float lse2 = rv ? a.lse[srow] * kLog2e : -INFINITY;
  const bool seen = lse2 != -INFINITY;
  const float delta = rv ? a.delta[srow] : 0.f;
  const int qp = rv ? (a.causal ? a.q_pos[row] : 0x7ffffffe) : (int)0x80000000;
  const int n_kt = (n_k + TILE - 1) / TILE;
  // key tiles whose first key is visible to the workgroup's last query (a
  // prefix: positions increase)
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

  // Two register sets: the set that holds tile j + 1 is written to LDS
  // during tile j and then receives tile j + 3, so every tile's loads have
  // about two tiles of compute to land.  Set indices are compile-time
  // (std::integral_constant), the loop steps two tiles at a time.
  u32x4 pk[2][4], pv[2][4];
  int ppos[2] = {0, 0};
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  const auto rk = rsrc(kbase, (uint32_t)n_k * 256u), rv_ = rsrc(vbase, (uint32_t)n_k * 256u);
  const auto rp = rsrc(a.k_pos, (uint32_t)n_k * 4u);
  auto fetch_tile = [&](auto set, int j) {
    constexpr int s = decltype(set)::value;
    fetch_rows(rk, j * TILE, pk[s], tid);  // keys past the block read as zeros
    fetch_rows(rv_, j * TILE, pv[s], tid);
    // raw position; the range and causal selects wait until it is written
    ppos[s] = __builtin_amdgcn_raw_buffer_load_b32(
        rp, (uint32_t)(j * TILE + (tid & (TILE - 1))) * 4u, 0, 0);
  };
  // slice w (0..12) of register set s into buffer b: K chunks (row and
  // transposing copies), then V chunks, then the key positions of tile j
  auto put_slice = [&](auto set, TileQ& b, int w, int j) {
    constexpr int s = decltype(set)::value;
    if (w < 8) {
      put_one(pk[s][w >> 1], (w & 1) ? nullptr : b.k_row, (w & 1) ? b.k_tr : nullptr, tid,
              w >> 1);
    } else if (w < 12) {
      put_one(pv[s][w - 8], b.v_row, nullptr, tid, w - 8);
    } else if (tid < TILE) {
      const int gk = j * TILE + tid;
      b.pos[tid] = gk < n_k ? (a.causal ? ppos[s] : (int)0x80000000) : 0x7fffffff;
    }
  };
  f32x16 dq[4] = {};
  const bool wave_ok = __builtin_amdgcn_ballot_w64(!(rv && seen)) == 0;
  const int qmin = __builtin_amdgcn_readfirstlane(qp);  // lane 0 holds the wave's first row
  if (n_iter > 0) {
    fetch_tile(Set0{}, 0);
#pragma unroll
    for (int w = 0; w < 13; ++w) put_slice(Set0{}, sm.t[0], w, 0);
    fetch_tile(Set1{}, 1);
    fetch_tile(Set0{}, 2);
  }
  __syncthreads();

  // tile j; `set` holds tile j + 1
  auto tile = [&](auto set, int j) {
    TileQ& cur = sm.t[j & 1];
    TileQ& nxt = sm.t[(j + 1) & 1];  // last read by tile j - 1, before the barrier
    // no mask when every row of the wave is valid, saw some key, and sees the
    // whole tile (positions increase, so the tile's last key decides)
    const bool full = wave_ok && __builtin_amdgcn_readfirstlane(cur.pos[TILE - 1]) <= qmin;
    auto body = [&](auto masked) {
      // A[kb][2 ks] = K rows, A[kb][2 ks + 1] = V rows of half kb; T[kb][4 t + db]
      // = transposed K for dQ^T += K^T dS^T.
      bf16x8 A[2][16], T[2][8];
      i32x4 pz[2][4];
      f32x16 S[2] = {}, P[2] = {};
      float X[2][16];
      bf16x8 ds[2][2];
      auto rdA = [&](int kb, int i) {
        A[kb][i] = row_operand((i & 1) ? cur.v_row : cur.k_row, L, kb, i >> 1);
      };
      auto rdT = [&](int kb, int i) { T[kb][i] = tr_operand(cur.k_tr, L, kb, i >> 2, i & 3); };
      auto mA = [&](int kb, int i) {
        if (i & 1)
          P[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[kb][i], dout[i >> 1], P[kb], 0, 0, 0);
        else
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[kb][i], q[i >> 1], S[kb], 0, 0, 0);
      };
      auto mT = [&](int kb, int i) {
        dq[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T[kb][i], ds[kb][i >> 2], dq[i & 3], 0,
                                                            0, 0);
      };
      auto valu = [&](int kb, int r) {
        float p;
        if constexpr (decltype(masked)::value) {
          const bool vis = pz[kb][r >> 2][r & 3] <= qp && seen;
          p = vis ? exp2f_(__builtin_fmaf(S[kb][r], a.c2, -lse2)) : 0.f;
        } else {
          p = exp2f_(__builtin_fmaf(S[kb][r], a.c2, -lse2));
        }
        X[kb][r] = p * (P[kb][r] - delta);
      };
      auto pack_ds = [&](int kb) {
  #pragma unroll
        for (int t = 0; t < 2; ++t)
  #pragma unroll
          for (int e = 0; e < 8; ++e) ds[kb][t][e] = (__bf16)X[kb][8 * t + e];
      };
  #pragma unroll
      for (int i = 0; i < AHEAD; ++i) rdA(0, i);
      read_half(cur.pos, 0, L.h, pz[0]);
      read_half(cur.pos, 1, L.h, pz[1]);
      RA_FENCE();
  #pragma unroll
      for (int i = 0; i < 16; ++i) {  // S, dP of half 0
        mA(0, i);
        if (i + AHEAD < 16) rdA(0, i + AHEAD); else rdA(1, i + AHEAD - 16);
        RA_FENCE();
      }
  #pragma unroll
      for (int i = 0; i < 16; ++i) {  // S, dP of half 1; dS of half 0
        mA(1, i);
        if (i + AHEAD < 16) rdA(1, i + AHEAD); else rdT(0, i + AHEAD - 16);
        valu(0, i);
        RA_FENCE();
      }
      pack_ds(0);
  #pragma unroll
      for (int i = 0; i < 8; ++i) {  // dQ from half 0; dS of half 1; tile j + 1 to LDS
        mT(0, i);
        if (i + AHEAD < 8) rdT(0, i + AHEAD); else rdT(1, i + AHEAD - 8);
        valu(1, 2 * i);
        valu(1, 2 * i + 1);
        put_slice(set, nxt, i, j + 1);
        RA_FENCE();
      }
      pack_ds(1);
  #pragma unroll
      for (int i = 0; i < 8; ++i) {  // dQ from half 1
        mT(1, i);
        if (i + AHEAD < 8) rdT(1, i + AHEAD);
        if (i < 5) put_slice(set, nxt, 8 + i, j + 1);
        if (i == 5) fetch_tile(set, j + 3);  // loads land two tiles later
        RA_FENCE();
      }
    };
    if (full)
      body(std::false_type{});
    else
      body(std::true_type{});
    __syncthreads();  // tile j + 1 is in place; tile j's buffer is free
  };
  for (int j = 0; j < n_iter; j += 2) {
    tile(Set1{}, j);
    if (j + 1 < n_iter) tile(Set0{}, j + 1);
  }
  // dq += this block's part, or dq = it (a.dq_write: the first block of a
  // whole-share backward, which then needs no zeroed dq)
  if (rv) {
    if (a.dq_write)
      store_rows<false>(a.dq + srow * D, dq, L.h, a.scale);
    else
      store_rows<true>(a.dq + srow * D, dq, L.h, a.scale);
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
hipError_t launch_backward_dq(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.n_q + bwd::ROWS - 1) / bwd::ROWS * a.h_q));
  hipLaunchKernelGGL(bwd::dq_kernel, grid, dim3(bwd::THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ra
