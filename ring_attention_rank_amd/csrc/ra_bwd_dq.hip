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
//  * dq kernel: 32 query rows (Q and dout in registers) walk the visible
//    64-key tiles: S^T = K Q^T and dP^T = V dout^T (K and V rows the A
//    operands), dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T (K read
//    transposed, dS^T packed to bf16 as the B operand straight from the
//    accumulators, as P^T feeds V^T P^T in the forward).
//  * dk/dv kernel (ra_bwd_dkv.hip): the mirror image.  32 keys (K and V rows
//    in registers) walk the query heads of their split of the key/value
//    head's group and the 64-query tiles that see those keys: S = Q K^T and
//    dP = dout V^T (Q and dout rows the A operands), dS = P (dP - delta),
//    dV^T += dout^T P and dK^T += Q^T dS (dout and Q read transposed).
//
// Both kernels run two waves per SIMD, each under 256 registers, as pairs
// of waves that own the same rows (here 32 queries, in ra_bwd_dkv.hip 32
// keys) and split the work between them.  Tiles go from HBM straight into
// LDS by buffer-load DMA, one copy each, in a swizzle that serves both the
// row reads and the transposing ds_read_b64_tr_b16 reads without bank
// conflicts.  Inside a phase the instructions are fenced in issue order,
// with the LDS operand reads a few MFMAs ahead of their use.
//
// This unit: the dq kernel and delta = rowsum(dout * out).  A workgroup of
// 8 waves owns 128 query rows; on each SIMD, with the tile's 64 keys in two
// halves of 32,
//  * the P wave (q and dout in registers): S^T_j = K_j q^T, p = exp(scale s
//    - lse) under the mask; p of key half 0 to LDS in fp32; for key half 1
//    also dP^T = V_j dout^T and dS^T = p (dP^T - delta), to LDS in bf16;
//  * the dS wave (dout and the dQ accumulator in registers): with the p of
//    tile j - 1's key half 0 from LDS, its dS^T from the dP^T it computed the
//    step before, and key half 1's dS^T from LDS, dQ^T += K_{j-1}^T dS^T;
//    then dP^T_j of key half 0 for the next step.
// Each wave issues 24 of the 48 MFMAs of a tile.  One barrier per step; K
// has three stages (j - 1, j, and j + 1 landing), V two, p and dS two.  The
// MFMA accumulators live in ordinary VGPRs (built with the VGPR form), so the
// VALU work reads them without moves.
#include "ra_bwd_common.h"

namespace ra {
namespace bwd {

constexpr int Q_THREADS = 512;

struct __attribute__((aligned(1024))) SmemQ {
  uint8_t k[3][TILE_BYTES];  // K tiles, one copy each (uswz layout): rows for S^T, transposed for dQ^T
  uint8_t v[2][TILE_BYTES];  // V tiles: rows for dP^T
  // p of a tile's key half 0, per wave pair, register group and lane: the P
  // wave's S^T accumulator layout, which is the dS wave's dP^T layout too
  f32x4 p[2][4][4][64];
  // dS^T of a tile's key half 1 in bf16, per wave pair, as the two B
  // operands of the dQ^T product (registers 0-7 and 8-15 of the layout)
  bf16x8 ds[2][4][2][64];
  int32_t pos[3][TILE];  // key positions as stored (keys past the block read as 0)
};

// LDS operand reads run this many MFMAs ahead of their use.
constexpr int Q_AHEAD = 3;

// dq kernel: one workgroup = 128 query rows of one head; a one-dimensional
// grid of n_qt128 * h_q workgroups.
__global__ __launch_bounds__(Q_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(const BwdArgs a) {
  __shared__ SmemQ sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pw = wave < 4;  // P wave (else dS wave)
  const int pair = wave & 3;
  const Lanes1 L(lane);
  int bx, head;  // heads that share a key/value head on one XCD
  xcd_split(blockIdx.x, a.h_q, bx, head);
  const int kvh = head / (a.h_q / a.h_kv);
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;
  const int row0_wg = bx * ROWS, row0 = row0_wg + pair * 32;
  const int row = row0 + L.col;
  const bool rv = row < n_q;
  const size_t srow = (size_t)head * n_q + row;

  // q (P wave) or dout (dS wave) in registers: the B operand of S^T or dP^T;
  // the P wave also holds dout for its half of dP^T
  const uint16_t* src = (const uint16_t*)(pw ? a.q : a.dout) + ((size_t)head * n_q) * D;
  const uint16_t* gsrc = (const uint16_t*)a.dout + ((size_t)head * n_q) * D;
  bf16x8 qg[8], dg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qg[ks] = rv ? *(const bf16x8*)(src + (size_t)row * D + ks * 16 + L.h * 8) : bf16x8{};
  if (pw) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      dg[ks] = rv ? *(const bf16x8*)(gsrc + (size_t)row * D + ks * 16 + L.h * 8) : bf16x8{};
  }
  // rows past n_q and rows that saw no key at all have lse = -inf: p = 0
  const float lse2 = rv ? a.lse[srow] * kLog2e : -INFINITY;
  const bool seen = lse2 != -INFINITY;
  const float delta = rv ? a.delta[srow] : 0.f;
  const int qp = rv ? (causal ? a.q_pos[row] : 0x7ffffffe) : (int)0x80000000;
  const int n_kt = (n_k + TILE - 1) / TILE;
  // key tiles whose first key is visible to the workgroup's last query (a
  // prefix: positions increase)
  int n_iter = n_kt;
  if (causal) {
    const int qmax = a.q_pos[min(row0_wg + ROWS, n_q) - 1];
    int cnt = 0;
    for (int j = lane; j < n_kt; j += 64) cnt += a.k_pos[j * TILE] <= qmax ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    n_iter = __builtin_amdgcn_readfirstlane(cnt);
  }
  // registers and row values land before any tile load is issued, so the
  // waits inside the loop only ever concern the next tile's DMA
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  const bool wave_ok = __builtin_amdgcn_ballot_w64(!(rv && seen)) == 0;
  const int qmin = __builtin_amdgcn_readfirstlane(qp);  // lane 0 holds the wave's first row

  // DMA of a tile: wave w moves rows 8 w .. 8 w + 7 of K and of V, load i
  // rows 8 w + 4 i + L / 16; lane L fills physical chunk L % 16 of its row
  // with logical chunk (L % 16) ^ uswz(row).  Wave 0 also moves the 64 key
  // positions.
  int dma_v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    dma_v[i] = (lane >> 4) * 256 + 16 * ((lane & 15) ^ (4 * (lane >> 4) | ((2 * wave + i) & 3)));
  const i32x4 rk = rsrc_words((const uint16_t*)a.k + ((size_t)kvh * n_k) * D, (uint32_t)n_k * 256u);
  const i32x4 rvv = rsrc_words((const uint16_t*)a.v + ((size_t)kvh * n_k) * D, (uint32_t)n_k * 256u);
  const i32x4 rp = rsrc_words(a.k_pos, (uint32_t)n_k * 4u);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&sm;
  auto dma_tile = [&](int j) {
    const uint32_t w = 8 * wave * 256;
    const int soff = (j * TILE + 8 * wave) * 256;
    dma_rows8(rk, lds0 + (uint32_t)offsetof(SmemQ, k) + (j % 3) * TILE_BYTES + w, dma_v[0],
              dma_v[1], soff);
    dma_rows8(rvv, lds0 + (uint32_t)offsetof(SmemQ, v) + (j & 1) * TILE_BYTES + w, dma_v[0],
              dma_v[1], soff);
    if (wave == 0)
      dma_words64(rp, lds0 + (uint32_t)offsetof(SmemQ, pos) + (j % 3) * TILE * 4, lane * 4,
                  j * TILE * 4);
  };
  // The P wave's mask decision for a tile: whole tile inside the block and
  // its last key visible to the wave's first row (positions increase), from
  // a scalar load one step ahead.
  auto tile_full = [&](int j) {
    const int last = j * TILE + TILE - 1;
    if (!wave_ok || last >= n_k) return false;
    return !causal || a.k_pos[last] <= qmin;
  };

  f32x16 acc[4] = {};  // dQ^T (dS wave)
  f32x16 sp[2];        // S^T of a tile's two 32-key halves (P wave); dP^T of half 0 (dS wave)
  f32x16 dp1;          // dP^T of key half 1 (P wave)
  bf16x8 op[16], tr[16];
  if (n_iter > 0) {
    dma_tile(0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  }
  __syncthreads();

  // 16 MFMAs sp[kb] += (rows of X, half kb) x qg; hook(n) after MFMA n
  auto rows_mfma = [&](const uint8_t* X, auto hook) {
    sp[0] = f32x16{};
    sp[1] = f32x16{};
#pragma unroll
    for (int n = 0; n < Q_AHEAD; ++n) op[n] = row_operand1(X, L, n >> 3, n & 7);
    RA_FENCE();
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      sp[n >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n], qg[n & 7], sp[n >> 3], 0, 0, 0);
      if (n + Q_AHEAD < 16) op[n + Q_AHEAD] = row_operand1(X, L, (n + Q_AHEAD) >> 3, (n + Q_AHEAD) & 7);
      hook(n);
      RA_FENCE();
    }
  };

  // 8 MFMAs out += (rows of X, key half kb) x B; hook(n) after MFMA n
  auto half_mfma = [&](const uint8_t* X, int kb, const bf16x8(&B)[8], f32x16& out, auto hook) {
    out = f32x16{};
#pragma unroll
    for (int n = 0; n < Q_AHEAD; ++n) op[n] = row_operand1(X, L, kb, n);
    RA_FENCE();
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n], B[n], out, 0, 0, 0);
      if (n + Q_AHEAD < 8) op[n + Q_AHEAD] = row_operand1(X, L, kb, n + Q_AHEAD);
      hook(n);
      RA_FENCE();
    }
  };

  // ---- the P wave: p of tile j's key half 0 into p slot j & 1, dS^T of
  // its key half 1 into dS slot j & 1
  auto p_step = [&](int j, auto masked) {
    constexpr bool M = decltype(masked)::value;
    const int32_t* pos = sm.pos[j % 3];
    f32x4* pb = &sm.p[j & 1][pair][0][lane];  // [group] stride 64
    auto pgroup = [&](int kb, int g) {
      f32x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float p;
        if constexpr (M) {
          const int kr = acc_row(kb, L.h, r);
          const bool vis = (!causal || pos[kr] <= qp) && seen && j * TILE + kr < n_k;
          p = vis ? exp2f_(__builtin_fmaf(sp[kb][r], a.c2, -lse2)) : 0.f;
        } else {
          p = exp2f_(__builtin_fmaf(sp[kb][r], a.c2, -lse2));
        }
        pv[e] = p;
      }
      return pv;
    };
    __builtin_amdgcn_s_setprio(1);  // its MFMAs first: the dS wave's fill its exponential tail
    rows_mfma(sm.k[j % 3], [&](int n) {
      if (n >= 8 && (n & 1)) pb[64 * ((n - 8) >> 1)] = pgroup(0, (n - 8) >> 1);
    });
    __builtin_amdgcn_s_setprio(0);
    // key half 1: dP^T beside its exponentials, then dS^T
    f32x4 p1[4];
    half_mfma(sm.v[j & 1], 1, dg, dp1, [&](int n) {
      if (n & 1) p1[n >> 1] = pgroup(1, n >> 1);
    });
    bf16x8 d1[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) d1[r >> 3][r & 7] = (__bf16)(p1[r >> 2][r & 3] * (dp1[r] - delta));
    sm.ds[j & 1][pair][0][lane] = d1[0];
    sm.ds[j & 1][pair][1][lane] = d1[1];
  };

  // ---- the dS wave: dS and dQ of tile j - 1 (its key half 0's dP^T in
  // sp[0], key half 1's dS^T from the P wave), then dP^T of tile j's key
  // half 0
  auto ds_step = [&](int j) {
    if (j > 0) {
      const int jp = j - 1;
      const f32x4* pb = &sm.p[jp & 1][pair][0][lane];
      const uint8_t* K = sm.k[jp % 3];
      bf16x8 ds[2][2];
      f32x4 pv[4];
      // dQ^T MFMA n: half n / 8, i = n % 8: d block i % 4, key group i / 4
      auto rd_t = [&](int n) { tr[n] = tr_operand1(K, L, n >> 3, (n & 7) >> 2, n & 3); };
#pragma unroll
      for (int g = 0; g < 4; ++g) pv[g] = pb[64 * g];
      ds[1][0] = sm.ds[jp & 1][pair][0][lane];
      ds[1][1] = sm.ds[jp & 1][pair][1][lane];
#pragma unroll
      for (int n = 0; n < Q_AHEAD; ++n) rd_t(n);
      RA_FENCE();
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ds[0][r >> 3][r & 7] = (__bf16)(pv[r >> 2][r & 3] * (sp[0][r] - delta));
      RA_FENCE();
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int i = n & 7;
        acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr[n], ds[n >> 3][i >> 2], acc[i & 3],
                                                             0, 0, 0);
        if (n + Q_AHEAD < 16) rd_t(n + Q_AHEAD);
        RA_FENCE();
      }
    }
    if (j < n_iter) half_mfma(sm.v[j & 1], 0, qg, sp[0], [](int) {});
  };

  // Each role runs its own copy of the loop (the same barriers in the same
  // order): steps j = 0 .. n_iter, the last one only the dS wave's tail.
  auto run = [&](auto is_p) {
    constexpr bool PW = decltype(is_p)::value;
    bool full_next = PW && n_iter > 0 && tile_full(0);
    for (int j = 0; j <= n_iter; ++j) {
      const bool more = j + 1 < n_iter;
      if (more) dma_tile(j + 1);
      if constexpr (PW) {
        if (j < n_iter) {
          const bool full = full_next;
          if (more) full_next = tile_full(j + 1);
          if (full)
            p_step(j, std::false_type{});
          else
            p_step(j, std::true_type{});
        }
      } else {
        ds_step(j);
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's part of tile j + 1 landed
      __syncthreads();  // tile j + 1, p_j and dS_j are in place; stages of j - 2 are free
    }
  };
  if (pw)
    run(std::true_type{});
  else
    run(std::false_type{});
  // dq += this block's part, or dq = it (a.dq_write: the first block of a
  // whole-share backward, which then needs no zeroed dq)
  if (!pw && rv) {
    if (a.dq_write)
      store_rows<false>(a.dq + srow * D, acc, L.h, a.scale);
    else
      store_rows<true>(a.dq + srow * D, acc, L.h, a.scale);
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
  hipLaunchKernelGGL(bwd::dq_kernel, grid, dim3(bwd::Q_THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ra
