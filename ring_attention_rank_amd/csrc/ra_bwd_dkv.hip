// Backward of one rank's share, bfloat16 with d_k = 128 on gfx950: the
// dk/dv kernel, the reduction of its head-group splits, and the launcher of
// the whole block step (the algorithm and the dq kernel are described in
// ra_bwd_dq.hip).  Its MFMA accumulators (dk, dv and two halves of S and
// dP: 256 values per lane) live in AGPRs.
#include "ra_bwd_common.h"

namespace ra {
namespace bwd {

// 1024-byte aligned: the second buffer keeps the 16-byte chunk alignment and
// the bank mapping of the swizzles.
struct __attribute__((aligned(1024))) TileKV {
  uint8_t q_row[TILE_BYTES];
  uint8_t q_tr[TILE_BYTES];
  uint8_t g_row[TILE_BYTES];
  uint8_t g_tr[TILE_BYTES];
  int32_t pos[TILE];
  float lse2[TILE];  // lse * log2(e); +inf where the row contributes nothing
  float delta[TILE];
  int32_t tile_ok;  // every query of the tile valid with a finite lse
};
// Two tile buffers: tile i is read from t[i & 1] while tile i + 1 is written
// into the other one, slice by slice between the MFMAs.
struct SmemKV {
  TileKV t[2];
};

// dk/dv kernel: one workgroup = 128 keys of one key/value head and one split
// of the query heads that read it; a one-dimensional grid of
// n_kt128 * h_kv * n_split workgroups.  Walks the split's heads and, per
// head, the query tiles that see these keys.  With one split it adds to dk,
// dv; with several, each split writes its partial sums to the workspace and
// a reduction adds them in a fixed order.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dkv_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) SmemKV sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lanes L(lane);
  const int n_split = a.n_split;
  int bx, by;  // one head-group split (its queries and dout) per XCD
  xcd_split(blockIdx.x, a.h_kv * n_split, bx, by);
  const int kvh = by / n_split, split = by % n_split;
  const int hps = a.h_q / a.h_kv / n_split;  // heads per split
  const int n_q = a.n_q, n_k = a.n_k;
  const int key0_wg = bx * ROWS, key0 = key0_wg + wave * 32;
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
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): k and v land before any tile load
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

  u32x4 pq[4], pg[4];
  int ppos = 0;
  float plse2 = 0.f, pdelta = 0.f;
  const auto rqp = rsrc(a.q_pos, (uint32_t)n_q * 4u);
  int tile_row0 = 0;  // first query row of the registered tile
  auto fetch_tile = [&](int i) {
    const int head = (kvh * n_split + split) * hps + i / n_t, t0 = first + i % n_t;
    const size_t hrow = (size_t)head * n_q;
    // queries past n_q read as zeros; every wave issues the same loads
    fetch_rows(rsrc((const uint16_t*)a.q + hrow * D, (uint32_t)n_q * 256u), t0 * TILE, pq, tid);
    fetch_rows(rsrc((const uint16_t*)a.dout + hrow * D, (uint32_t)n_q * 256u), t0 * TILE, pg,
               tid);
    const uint32_t o = (uint32_t)(t0 * TILE + (tid & (TILE - 1))) * 4u;
    // raw per-row values; the range selects wait until they are written
    ppos = __builtin_amdgcn_raw_buffer_load_b32(rqp, o, 0, 0);
    plse2 = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.lse + hrow, (uint32_t)n_q * 4u), o, 0, 0));
    pdelta = __builtin_bit_cast(
        float,
        __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.delta + hrow, (uint32_t)n_q * 4u), o, 0, 0));
    tile_row0 = t0 * TILE;
  };
  // slice w (0..16) of the registered tile into buffer b: Q and dout chunks
  // (row and transposing copies), then the per-row values and the tile flag
  auto put_slice = [&](TileKV& b, int w) {
    if (w < 16) {
      const u32x4& x = (w < 8) ? pq[(w & 7) >> 1] : pg[(w & 7) >> 1];
      uint8_t* row = (w < 8) ? b.q_row : b.g_row;
      uint8_t* tr = (w < 8) ? b.q_tr : b.g_tr;
      put_one(x, (w & 1) ? nullptr : row, (w & 1) ? tr : nullptr, tid, (w & 7) >> 1);
    } else {
      const bool ok = tile_row0 + (tid & (TILE - 1)) < n_q;
      const float l = ok ? plse2 : -INFINITY;
      // log2-domain lse; +inf for rows past n_q and rows that saw no key, so
      // that their probabilities come out as exp2(-inf) = 0
      const float l2 = l != -INFINITY ? l * kLog2e : INFINITY;
      if (tid < TILE) {
        b.pos[tid] = ok ? (a.causal ? ppos : 0x7ffffffe) : (int)0x80000000;
        b.lse2[tid] = l2;
        b.delta[tid] = ok ? pdelta : 0.f;
      }
      if (wave == 0) {  // wave 0 holds the tile's 64 rows, one per lane
        const bool all = __builtin_amdgcn_ballot_w64(l2 != INFINITY) == ~0ull;
        if (lane == 0) b.tile_ok = all ? 1 : 0;
      }
    }
  };
  f32x16 dk[4] = {}, dv[4] = {};
  const int kmax_w = __builtin_amdgcn_readlane(kp, 31);  // lane 31 holds the wave's last key
  if (total > 0) {
    fetch_tile(0);
#pragma unroll
    for (int w = 0; w < 17; ++w) put_slice(sm.t[0], w);
    // a tile index past the split's last maps to another head: never fetched
    if (total > 1) fetch_tile(1);
  }
  __syncthreads();

  for (int i_tile = 0; i_tile < total; ++i_tile) {
    TileKV& cur = sm.t[i_tile & 1];
    TileKV& nxt = sm.t[(i_tile + 1) & 1];  // last read by the previous tile, before the barrier
    const bool more = i_tile + 2 < total;
    // no causal mask when every query of the tile is valid with a finite lse
    // and sees every key of the wave (the tile's first query and the wave's
    // last key decide)
    const bool full = __builtin_amdgcn_readfirstlane(cur.tile_ok) &&
                      kmax_w <= __builtin_amdgcn_readfirstlane(cur.pos[0]);
    // A[qb][2 ks] = Q rows, A[qb][2 ks + 1] = dout rows of half qb;
    // TG/TQ[qb][4 t + db] = transposed dout / Q for dV^T += dout^T P and
    // dK^T += Q^T dS.
    bf16x8 A[2][16], TG[2][8], TQ[2][8];
    i32x4 pz[2][4];
    f32x4 lz[2][4], dz[2][4];
    f32x16 S[2] = {}, P[2] = {};
    bf16x8 pp[2][2], ds[2][2];
    auto rdA = [&](int qb, int i) {
      A[qb][i] = row_operand((i & 1) ? cur.g_row : cur.q_row, L, qb, i >> 1);
    };
    auto rdT = [&](int qb, int i) {
      const int j = i >> 1;
      if (i & 1)
        TQ[qb][j] = tr_operand(cur.q_tr, L, qb, j >> 2, j & 3);
      else
        TG[qb][j] = tr_operand(cur.g_tr, L, qb, j >> 2, j & 3);
    };
    // per-row values of accumulator registers 4 g .. 4 g + 3 of half qb
    auto rd_grp = [&](int qb, int g) {
      const int o = 32 * qb + 8 * L.h + 4 * (g & 1) + 16 * (g >> 1);
      pz[qb][g] = *(const i32x4*)(cur.pos + o);
      lz[qb][g] = *(const f32x4*)(cur.lse2 + o);
      dz[qb][g] = *(const f32x4*)(cur.delta + o);
    };
    auto mA = [&](int qb, int i) {
      if (i & 1)
        P[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[qb][i], vr[i >> 1], P[qb], 0, 0, 0);
      else
        S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[qb][i], kr[i >> 1], S[qb], 0, 0, 0);
    };
    auto mT = [&](int qb, int i) {
      const int j = i >> 1;
      if (i & 1)
        dk[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(TQ[qb][j], ds[qb][j >> 2], dk[j & 3],
                                                            0, 0, 0);
      else
        dv[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(TG[qb][j], pp[qb][j >> 2], dv[j & 3],
                                                            0, 0, 0);
    };
    // p and ds of registers 2 j, 2 j + 1 of half qb, converted to bf16 as a
    // pair
    auto valu2 = [&](int qb, int j) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = 2 * j + u;
        // rows past n_q and rows that saw no key carry l2 = +inf: p = 0
        float p = exp2f_(__builtin_fmaf(S[qb][r], a.c2, -lz[qb][r >> 2][r & 3]));
        if (!full && kp > pz[qb][r >> 2][r & 3]) p = 0.f;
        pp[qb][r >> 3][r & 7] = (__bf16)p;
        ds[qb][r >> 3][r & 7] = (__bf16)(p * (P[qb][r] - dz[qb][r >> 2][r & 3]));
      }
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) rdA(0, i);
    rd_grp(0, 0);
    RA_FENCE();
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // S, dP of half 0; tile i + 1 into the other buffer
      mA(0, i);
      if (i + 4 < 16) rdA(0, i + 4); else rdA(1, i - 12);
      put_slice(nxt, i);
      RA_FENCE();
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // S, dP of half 1; P, dS of half 0
      mA(1, i);
      if (i + 4 < 16) rdA(1, i + 4); else rdT(0, i - 12);
      if (i == 0) put_slice(nxt, 16);
      if (i == 1 && more) fetch_tile(i_tile + 2);
      if ((i & 3) == 1) {  // starting row group i / 4: fetch the next one
        if (i < 12) rd_grp(0, (i >> 2) + 1); else rd_grp(1, 0);
      }
      if (i & 1) valu2(0, i >> 1);
      RA_FENCE();
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // dV, dK from half 0; P, dS of half 1
      mT(0, i);
      if (i + 4 < 16) rdT(0, i + 4); else rdT(1, i - 12);
      if ((i & 3) == 1 && i < 12) rd_grp(1, (i >> 2) + 1);
      if (i & 1) valu2(1, i >> 1);
      RA_FENCE();
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // dV, dK from half 1
      mT(1, i);
      if (i + 4 < 16) rdT(1, i + 4);
      RA_FENCE();
    }
    __syncthreads();  // tile i + 1 is in place; tile i's buffer is free
  }
  if (kv) {
    float* ddk = a.dk;
    float* ddv = a.dv;
    if (n_split > 1) {  // partial sums of this split
      const size_t part = (size_t)a.h_kv * n_k * D;
      ddk = a.ws + (size_t)split * part;
      ddv = a.ws + (size_t)(n_split + split) * part;
    }
    if (n_split > 1 || a.overwrite) {
      store_rows<false>(ddk + skey * D, dk, L.h, a.scale);
      store_rows<false>(ddv + skey * D, dv, L.h, 1.f);
    } else {  // added to the caller's (travelling) dk, dv
      store_rows<true>(ddk + skey * D, dk, L.h, a.scale);
      store_rows<true>(ddv + skey * D, dv, L.h, 1.f);
    }
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
  // Split the head group until the dk/dv grid has about 1024 workgroups (4
  // per compute unit), over divisors of the group size.
  const int grp = h_q / h_kv, tiles = (n_k + bwd::ROWS - 1) / bwd::ROWS * h_kv;
  int g = 1;
  while (g < grp && (int64_t)tiles * g < 1024) {
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
  hipLaunchKernelGGL(bwd::dkv_kernel, grid, dim3(bwd::THREADS), 0, stream, a);
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
