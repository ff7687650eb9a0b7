// Backward of one rank's share, bfloat16 with d_k = 128 on gfx950: the
// dk/dv kernel, the reduction of its head-group splits, and the launcher of
// the whole block step (the algorithm and the dq kernel are described in
// ra_bwd_dq.hip).
//
// Two waves per SIMD.  A workgroup owns 128 keys and runs 8 waves: on every
// SIMD a pair of waves that own the same 32 keys and split the work of a
// query tile between them,
//  * the P wave (K rows in registers): S = Q K^T, p = exp(scale s - lse)
//    under the mask, then dV^T += dout^T P;
//  * the dS wave (V rows in registers): dP = dout V^T, then, with the pair's
//    p read back from LDS, dS = p (dP - delta) and dK^T += Q^T dS.
// Each wave holds one 32-key x 128 accumulator (dV or dK), so both fit in 256
// registers, and while one wave of a SIMD works through its exponentials or
// its dS the other keeps the matrix pipe busy.
//
// Q and dout tiles go from HBM straight into LDS (one copy each, in a layout
// that serves both the row reads and the transposing reads).  The two waves
// of a pair run skewed, so that in each phase one of them reads rows, the
// other transposes, and one of them has VALU work beside its MFMAs:
//   phase A of tile i:  P wave  S_i = Q_i K^T (rows of Q_i), p -> LDS
//                       dS wave dK^T += Q_{i-1}^T dS_{i-1} (Q_{i-1} transposed)
//   phase B of tile i:  P wave  dV^T += dout_i^T P_i (dout_i transposed)
//                       dS wave dP_i = dout_i V^T (rows of dout_i), dS_i
// with a barrier after each phase.  Q therefore has three stages (i - 1, i,
// and i + 1 landing), dout two; the DMA of tile i + 1 is issued when tile i
// starts.
#include "ra_bwd_common.h"

namespace ra {
namespace bwd {

constexpr int KV_THREADS = 512;

struct RowVals {
  int32_t pos[TILE];
  float lse2[TILE];  // lse * log2(e); +inf where the row contributes nothing
  float delta[TILE];
};
struct __attribute__((aligned(1024))) SmemKV {
  uint8_t q[3][TILE_BYTES];  // Q tiles, one copy each (uswz layout)
  uint8_t g[2][TILE_BYTES];  // dout tiles
  // p of the current tile, per wave pair, half, register group and lane: the
  // P wave's accumulator layout, which is the dS wave's dP layout too
  f32x4 p[4][2][4][64];
  RowVals rows[2];
};

// LDS operand reads run this many MFMAs ahead of their use.
constexpr int KV_AHEAD = 3;

// dk/dv kernel: one workgroup = 128 keys of one key/value head and one split
// of the query heads that read it; a one-dimensional grid of
// n_kt128 * h_kv * n_split workgroups.  Walks the split's heads and, per
// head, the query tiles that see these keys.  With one split it adds to (or,
// overwrite, writes) dk, dv; with several, each split writes its partial sums
// to the workspace and a reduction adds them in a fixed order.
__global__ __launch_bounds__(KV_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkv_kernel(const BwdArgs a) {
  __shared__ SmemKV sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pw = wave < 4;  // P wave (else dS wave)
  const int pair = wave & 3;
  const Lanes1 L(lane);
  const int n_split = a.n_split;
  int bx, by;  // one head-group split (its queries and dout) per XCD
  xcd_split(blockIdx.x, a.h_kv * n_split, bx, by);
  const int kvh = by / n_split, split = by % n_split;
  const int hps = a.h_q / a.h_kv / n_split;  // heads per split
  const int n_q = a.n_q, n_k = a.n_k;
  const int key0_wg = bx * ROWS, key0 = key0_wg + pair * 32;
  const int key = key0 + L.col;
  const bool kv = key < n_k;
  const size_t skey = (size_t)kvh * n_k + key;

  // K rows (P wave) or V rows (dS wave): the B operand of S or dP
  const uint16_t* src = (const uint16_t*)(pw ? a.k : a.v) + ((size_t)kvh * n_k) * D;
  bf16x8 kvr[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    kvr[ks] = kv ? *(const bf16x8*)(src + (size_t)key * D + ks * 16 + L.h * 8) : bf16x8{};
  // this lane's key position; keys past the block see nothing
  const int kp = kv ? (a.causal ? a.k_pos[key] : (int)0x80000000) : 0x7fffffff;
  // query tiles that see any of the workgroup's keys form a suffix
  const int n_qt = (n_q + TILE - 1) / TILE;
  int first = 0;
  if (a.causal && n_qt > 0) {
    const int kmin = a.k_pos[key0_wg];
    int cnt = 0;  // tiles whose last query precedes kmin
    for (int t = lane; t < n_qt; t += 64)
      cnt += a.q_pos[min(t * TILE + TILE, n_q) - 1] < kmin ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    first = __builtin_amdgcn_readfirstlane(cnt);
  }
  const int n_t = n_qt - first, total = hps * n_t;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): registers and positions land first
  const int kmax_w = __builtin_amdgcn_readlane(kp, 31);  // lane 31 holds the wave's last key

  // DMA of a tile: wave w moves rows 8 w .. 8 w + 7 of Q and of dout, load i
  // rows 8 w + 4 i + L / 16; lane L fills physical chunk L % 16 of its row
  // with logical chunk (L % 16) ^ uswz(row).
  int dma_v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    dma_v[i] = (lane >> 4) * 256 + 16 * ((lane & 15) ^ (4 * (lane >> 4) | ((2 * wave + i) & 3)));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&sm;
  // per-row values of a tile (wave 0: one row per lane)
  int ppos = 0;
  float plse = 0.f, pdelta = 0.f;
  int row_t0 = 0;
  auto tile_of = [&](int i, int& head, int& t0) {
    head = (kvh * n_split + split) * hps + i / n_t;
    t0 = first + i % n_t;
  };
  auto dma_tile = [&](int i) {
    int head, t0;
    tile_of(i, head, t0);
    const size_t hrow = (size_t)head * n_q;
    const uint32_t w = 8 * wave * 256;
    const int soff = (t0 * TILE + 8 * wave) * 256;
    dma_rows8(rsrc_words((const uint16_t*)a.q + hrow * D, (uint32_t)n_q * 256u),
              lds0 + (uint32_t)offsetof(SmemKV, q) + (i % 3) * TILE_BYTES + w, dma_v[0],
              dma_v[1], soff);
    dma_rows8(rsrc_words((const uint16_t*)a.dout + hrow * D, (uint32_t)n_q * 256u),
              lds0 + (uint32_t)offsetof(SmemKV, g) + (i & 1) * TILE_BYTES + w, dma_v[0],
              dma_v[1], soff);
  };
  // wave 0 loads them late in a tile (short live range), and writes them
  // after its vmcnt(0)
  auto load_rows = [&](int i) {
    if (wave == 0) {
      int head, t0;
      tile_of(i, head, t0);
      const size_t hrow = (size_t)head * n_q;
      const uint32_t o = (uint32_t)(t0 * TILE + lane) * 4u;
      ppos = __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.q_pos, (uint32_t)n_q * 4u), o, 0, 0);
      plse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rsrc(a.lse + hrow, (uint32_t)n_q * 4u), o, 0, 0));
      pdelta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rsrc(a.delta + hrow, (uint32_t)n_q * 4u), o, 0, 0));
      row_t0 = t0 * TILE;
    }
  };
  auto put_rows = [&](RowVals& b) {
    if (wave == 0) {
      const bool ok = row_t0 + lane < n_q;
      const float l = ok ? plse : -INFINITY;
      // log2-domain lse; +inf for rows past n_q and rows that saw no key, so
      // that their probabilities come out as exp2(-inf) = 0
      const float l2 = l != -INFINITY ? l * kLog2e : INFINITY;
      b.pos[lane] = ok ? (a.causal ? ppos : 0x7ffffffe) : (int)0x80000000;
      b.lse2[lane] = l2;
      b.delta[lane] = ok ? pdelta : 0.f;
    }
  };
  // The P wave's mask decision for a tile: its first query's position, read
  // with a scalar load one tile ahead (no LDS round trip before the tile's
  // first MFMA).  Rows past n_q and rows that saw no key need no mask: their
  // l2 = +inf gives p = 0 either way.
  auto tile_pos0 = [&](int i) {
    int head, t0;
    tile_of(i, head, t0);
    return a.causal ? a.q_pos[t0 * TILE] : 0x7ffffffe;
  };

  f32x16 acc[4] = {};  // dV^T (P wave) or dK^T (dS wave)
  f32x16 sp[2];        // S (P wave) or dP (dS wave) of the tile's two 32-query halves
  bf16x8 bop[2][2];    // P_i (P wave) or dS_{i-1} / dS_i (dS wave) in bf16: B operands
  bf16x8 op[16];
  f32x4* pbuf = &sm.p[pair][0][0][lane];  // [half][group] stride 64
  auto row_off = [&](int qb, int g) { return 32 * qb + 8 * L.h + 4 * (g & 1) + 16 * (g >> 1); };

  // 16 MFMAs sp[qb] = (rows of X) x kvr, half 0 then half 1; hook(n) runs
  // after MFMA n (the VALU work of half 0 overlaps the MFMAs of half 1).
  auto rows_mfma = [&](const uint8_t* X, auto hook) {
    sp[0] = f32x16{};
    sp[1] = f32x16{};
#pragma unroll
    for (int n = 0; n < KV_AHEAD; ++n) op[n] = row_operand1(X, L, n >> 3, n & 7);
    RA_FENCE();
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      sp[n >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n], kvr[n & 7], sp[n >> 3], 0, 0, 0);
      if (n + KV_AHEAD < 16) op[n + KV_AHEAD] = row_operand1(X, L, (n + KV_AHEAD) >> 3, (n + KV_AHEAD) & 7);
      hook(n);
      RA_FENCE();
    }
  };
  // 16 MFMAs acc[db] += (Y transposed) x bop; MFMA n: half n / 8, j = n % 8:
  // d block j % 4, row group t = j / 4.
  auto tr_mfma = [&](const uint8_t* Y) {
    auto rd = [&](int n) {
      const int j = n & 7;
      op[n] = tr_operand1(Y, L, n >> 3, j >> 2, j & 3);
    };
#pragma unroll
    for (int n = 0; n < KV_AHEAD; ++n) rd(n);
    RA_FENCE();
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int j = n & 7;
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n], bop[n >> 3][j >> 2], acc[j & 3],
                                                           0, 0, 0);
      if (n + KV_AHEAD < 16) rd(n + KV_AHEAD);
      RA_FENCE();
    }
  };

  // ---- P wave, phase A: S_i, p = exp2(c2 s - lse2) under the mask, to LDS
  // (fp32) and to bop (bf16).  Per-row values are read a section or more
  // ahead of their use (the fences keep the order as written).
  auto p_phase_a = [&](const RowVals& rv, const uint8_t* X, auto masked) {
    constexpr bool M = decltype(masked)::value;
    f32x4 lz[2][4];
    i32x4 pz[2][4];
    auto rd_rows = [&](int qb, int g) {
      lz[qb][g] = *(const f32x4*)(rv.lse2 + row_off(qb, g));
      if constexpr (M) pz[qb][g] = *(const i32x4*)(rv.pos + row_off(qb, g));
    };
    auto pgroup = [&](int qb, int g) {
      f32x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        // rows past n_q and rows that saw no key carry l2 = +inf: p = 0
        float p = exp2f_(__builtin_fmaf(sp[qb][r], a.c2, -lz[qb][g][e]));
        if constexpr (M) p = kp > pz[qb][g][e] ? 0.f : p;
        pv[e] = p;
        bop[qb][r >> 3][r & 7] = (__bf16)p;
      }
      pbuf[64 * (4 * qb + g)] = pv;
    };
#pragma unroll
    for (int g = 0; g < 4; ++g) rd_rows(0, g);
    __builtin_amdgcn_s_setprio(1);  // its MFMAs first: the dS wave's fill the VALU tail
    rows_mfma(X, [&](int n) {
      if (n >= 8 && !(n & 1)) rd_rows(1, (n - 8) >> 1);
      if (n >= 8 && (n & 1)) pgroup(0, (n - 8) >> 1);
    });
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) pgroup(1, g);
  };
  // ---- dS wave, phase B: dP_i, then dS_i = p (dP - delta) into bop
  auto ds_phase_b = [&](const RowVals& rv, const uint8_t* X) {
    f32x4 pv[2][4], dz[2][4];
    auto rd = [&](int qb, int g) {
      pv[qb][g] = pbuf[64 * (4 * qb + g)];
      dz[qb][g] = *(const f32x4*)(rv.delta + row_off(qb, g));
    };
    auto dsgroup = [&](int qb, int g) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        bop[qb][r >> 3][r & 7] = (__bf16)(pv[qb][g][e] * (sp[qb][r] - dz[qb][g][e]));
      }
    };
#pragma unroll
    for (int g = 0; g < 4; ++g) rd(0, g);
    __builtin_amdgcn_s_setprio(1);
    rows_mfma(X, [&](int n) {
      if (n >= 8 && !(n & 1)) rd(1, (n - 8) >> 1);
      if (n >= 8 && (n & 1)) dsgroup(0, (n - 8) >> 1);
    });
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) dsgroup(1, g);
  };

  if (total > 0) {
    dma_tile(0);
    load_rows(0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    put_rows(sm.rows[0]);
  }
  __syncthreads();

  // Each role runs its own copy of the loop (the same barriers in the same
  // order), so each keeps its accumulators in place.
  auto run = [&](auto is_p) {
    constexpr bool PW = decltype(is_p)::value;
    int pos0 = (PW && total > 0) ? tile_pos0(0) : 0;
    for (int i = 0; i < total; ++i) {
      const bool more = i + 1 < total;
      const RowVals& rv = sm.rows[i & 1];
      const uint8_t* q_cur = sm.q[i % 3];
      const uint8_t* g_cur = sm.g[i & 1];
      if (more) dma_tile(i + 1);
      // ---- phase A
      if constexpr (PW) {
        // no causal mask when every query of the tile sees every key of the
        // wave (positions increase: the tile's first query and the wave's
        // last key decide)
        const bool full = kmax_w <= pos0;
        if (more) pos0 = tile_pos0(i + 1);
        if (full)
          p_phase_a(rv, q_cur, std::false_type{});
        else
          p_phase_a(rv, q_cur, std::true_type{});
      } else {
        if (i > 0) tr_mfma(sm.q[(i + 2) % 3]);  // dK from tile i - 1
      }
      __syncthreads();  // the pair's p is in LDS
      if (more) load_rows(i + 1);
      // ---- phase B
      if constexpr (PW)
        tr_mfma(g_cur);  // dV
      else
        ds_phase_b(rv, g_cur);
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's part of tile i + 1 landed
      if (more) put_rows(sm.rows[(i + 1) & 1]);
      __syncthreads();  // tile i + 1 is in place; tile i - 1's Q stage and p are free
    }
    // the dS wave's last dK (its Q stage is not overwritten any more)
    if constexpr (!PW) {
      if (total > 0) tr_mfma(sm.q[(total - 1) % 3]);
    }
  };
  if (pw)
    run(std::true_type{});
  else
    run(std::false_type{});
  if (kv) {
    // the P wave stores dv, the dS wave dk
    float* dst = pw ? a.dv : a.dk;
    const float mul = pw ? 1.f : a.scale;
    if (n_split > 1) {  // partial sums of this split
      const size_t part = (size_t)a.h_kv * n_k * D;
      dst = a.ws + (size_t)((pw ? n_split : 0) + split) * part;
    }
    if (n_split > 1 || a.overwrite)
      store_rows<false>(dst + skey * D, acc, L.h, mul);
    else  // added to the caller's (travelling) dk, dv
      store_rows<true>(dst + skey * D, acc, L.h, mul);
  }
}

// dk, dv += sums of the splits' partials, split 0 first.
__global__ __launch_bounds__(256) void reduce_kernel(const float* ws, float* dk, float* dv,
                                                     int64_t n4, int n_split, int overwrite) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* w = (const f32x4*)ws;
  f32x4 sk = w[i], sv = w[(int64_t)n_split * n4 + i];
  for (int s = 1; s < n_split; ++s) {
    sk += w[(int64_t)s * n4 + i];
    sv += w[(int64_t)(n_split + s) * n4 + i];
  }
  // the block's part is summed first, then added once to the caller's value
  // (or written, overwrite)
  if (overwrite) {
    ((f32x4*)dk)[i] = sk;
    ((f32x4*)dv)[i] = sv;
  } else {
    ((f32x4*)dk)[i] = ((const f32x4*)dk)[i] + sk;
    ((f32x4*)dv)[i] = ((const f32x4*)dv)[i] + sv;
  }
}

}  // namespace bwd

int backward_splits(int n_k, int h_q, int h_kv) {
  // Split the head group until the dk/dv grid has about 512 workgroups (two
  // rounds of one workgroup per compute unit), over divisors of the group
  // size.  More splits fill the rounds no better and add partial sums for
  // the reduction to read.
  const int grp = h_q / h_kv, tiles = (n_k + bwd::ROWS - 1) / bwd::ROWS * h_kv;
  int g = 1;
  while (g < grp && (int64_t)tiles * g < 512) {
    int nx = g + 1;
    while (grp % nx) ++nx;
    g = nx;
  }
  return g;
}

size_t backward_ws_bytes(int n_k, int h_q, int h_kv) {
  const int g = backward_splits(n_k, h_q, h_kv);
  return g > 1 ? (size_t)2 * g * h_kv * n_k * bwd::D * sizeof(float) : 0;
}

// dk/dv kernel and, with a head-group split, the reduction of its partials.
hipError_t launch_backward_dkv(const BwdArgs& a, hipStream_t stream) {
  if (a.n_k == 0) return hipSuccess;
  dim3 grid((unsigned)((a.n_k + bwd::ROWS - 1) / bwd::ROWS * a.h_kv * a.n_split));
  hipLaunchKernelGGL(bwd::dkv_kernel, grid, dim3(bwd::KV_THREADS), 0, stream, a);
  if (a.n_split > 1) {
    const int64_t n4 = (int64_t)a.h_kv * a.n_k * bwd::D / 4;
    hipLaunchKernelGGL(bwd::reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                       stream, a.ws, a.dk, a.dv, n4, a.n_split, a.overwrite);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  if (a.n_q > 0) {
    const hipError_t e = launch_backward_dq(a, stream);
    if (e != hipSuccess) return e;
  }
  return launch_backward_dkv(a, stream);
}

}  // namespace ra
