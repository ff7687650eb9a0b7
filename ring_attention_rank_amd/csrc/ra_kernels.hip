// HIP kernels for one ring step of causal attention on gfx950 (MI355X).
//
// What a step computes (Zero to Frontier, "distributed/context-expert",
// section "Splitting the sequence, and the one layer that objects"): every
// local query meets one key/value block; its running maximum, running sum of
// exponentials and running weighted sum of values are rescaled whenever the
// block brings a larger score, then the block's terms are added.  Done one
// 64-key tile at a time inside the block, this is the blockwise online
// softmax the "Context Parallelism (CP)" concept page names in "Key math /
// How it works".
//
// Mapping onto CDNA4:
//  * A workgroup is 4 waves (one per SIMD) and owns 256 consecutive query
//    rows of one head; each wave owns 64 rows as two 32-row MFMA blocks.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (fp32 inputs: v_mfma_f32_32x32x2_f32).  K is the A operand, read from
//    LDS; Q is the B operand and stays in registers for the whole block.  In
//    the S^T accumulator every lane holds one query column and 16 keys, so
//    row max and row sum are in-lane, plus one v_permlane32_swap between the
//    two half-waves.
//  * The accumulator rows are mapped to keys through sigma (swap of index
//    bits 2 and 3), which makes each half-wave's 8 P values of a 16-key step
//    8 consecutive keys.  P^T then feeds the PV MFMA (O^T = V^T P^T) as the B
//    operand straight from the accumulators, and V^T is staged in LDS so the
//    A operand is one 16-byte read.
//  * K and V^T tiles are double-buffered in LDS (rows padded by 16 bytes
//    against bank conflicts), loaded from HBM with 16-byte loads one tile
//    ahead.
//  * Tiles are classified from the explicit positions: skipped (no visible
//    pair), full (every pair visible) or masked (diagonal or ragged).  Only
//    masked tiles compare positions.
//  * Units (query tile, head) are launched heaviest first: positions increase
//    within a rank, so later query tiles see at least as many keys.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPosHidden = 0x7fffffff;        // key slot past the block's end
constexpr int kPosAlways = (int)0x80000000;   // key visible to every row (non-causal)
constexpr int kPosRowNone = (int)0x80000000;  // query row past the end: sees no causal key
constexpr int kPosRowAll = 0x7ffffffe;        // non-causal query row

// Accumulator row i of a 32-key block holds key sigma(i): bits 2 and 3 swapped.
__device__ __forceinline__ int sigma(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Max / sum of a value with the lane 32 away (the other half-wave).
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int wave_sum_i(int x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Element-type traits.  Each provides: the Q registers, staging a K/V tile
// from HBM into registers and then into LDS, S^T = K Q^T for one tile and
// O^T += V^T P^T for one tile.
// ---------------------------------------------------------------------------

// bfloat16 inputs, v_mfma_f32_32x32x16_bf16.
template <int D>
struct TraitsBf16 {
  typedef uint16_t Elem;  // bfloat16 bits in HBM
  typedef uint16_t LA;    // LDS element of the K stage
  typedef uint16_t LB;    // LDS element of the V^T stage
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int KCH = kKeysPerTile * CPR / 256;   // K chunks per thread per tile
  static constexpr int NV = KCH;                         // V keys per thread per tile
  static constexpr int KS = D / 16;                      // QK k-steps
  static constexpr int DB = D / 32;                      // 32-wide d blocks of O^T
  static constexpr int KSTR = D + 8;                     // padded K row (elements)
  static constexpr int VSTR = kKeysPerTile + 8;          // padded V^T row (elements)
  static constexpr int A_ELEMS = kKeysPerTile * KSTR;    // K stage
  static constexpr int B_ELEMS = D * VSTR;               // V^T stage

  struct Regs {
    u32x4 k[KCH];
    u32x4 v[NV];
  };
  struct Q {
    bf16x8 r[2][KS];
  };

  // Rows are padded by 16 bytes: 16 consecutive rows read at the same column
  // then fall on 16 distinct groups of 4 banks, and every offset used inside
  // the tile loops is a compile-time immediate.
  static __device__ __forceinline__ int k_off(int key, int chunk) { return key * KSTR + chunk * 8; }
  static __device__ __forceinline__ int vt_off(int d, int key) { return d * VSTR + key; }

  static __device__ __forceinline__ void load_q(Q& q, const void* qbase, int row0, int n_q,
                                                int col, int h) {
    const uint16_t* Qp = (const uint16_t*)qbase;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      int r = row0 + qb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (r < n_q) {
          q.r[qb][ks] = *(const bf16x8*)(Qp + (size_t)r * D + ks * 16 + h * 8);
        } else {
          q.r[qb][ks] = bf16x8{};
        }
      }
    }
  }

  static __device__ __forceinline__ void load_tile(Regs& g, const void* kbase, const void* vbase,
                                                   int j0, int n_k, int tid) {
    const uint16_t* Kp = (const uint16_t*)kbase;
    const uint16_t* Vp = (const uint16_t*)vbase;
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int c = tid + 256 * p;
      int key = c / CPR, dc = c % CPR;
      int gk = j0 + key;
      g.k[p] = gk < n_k ? *(const u32x4*)(Kp + (size_t)gk * D + dc * 8) : u32x4{0, 0, 0, 0};
    }
    constexpr int KG = kKeysPerTile / NV;  // key groups per tile
    int kg = tid % KG, dc = tid / KG;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int gk = j0 + kg * NV + i;
      g.v[i] = gk < n_k ? *(const u32x4*)(Vp + (size_t)gk * D + dc * 8) : u32x4{0, 0, 0, 0};
    }
  }

  static __device__ __forceinline__ void store_tile(const Regs& g, uint16_t* sk, uint16_t* svt,
                                                    int tid) {
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int c = tid + 256 * p;
      int key = c / CPR, dc = c % CPR;
      *(u32x4*)(sk + k_off(key, dc)) = g.k[p];
    }
    // Transpose the thread's NV keys x 8 d block into V^T rows d = 8*dc + e.
    // Lanes of one store cover consecutive keys of one row (and the next 32
    // lanes the row 8 further, 32 banks away), so the stores do not conflict.
    constexpr int KG = kKeysPerTile / NV;
    int kg = tid % KG, dc = tid / KG;
    int key0 = kg * NV;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int w = e >> 1;
      bool hi = e & 1;
      int d = dc * 8 + e;
      uint32_t a0 = g.v[0][w], a1 = g.v[1][w];
      uint32_t lo = hi ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
      uint16_t* dst = svt + vt_off(d, key0);
      if constexpr (NV == 4) {
        uint32_t a2 = g.v[2][w], a3 = g.v[3][w];
        uint32_t up = hi ? ((a2 >> 16) | (a3 & 0xffff0000u)) : ((a2 & 0xffffu) | (a3 << 16));
        *(u32x2*)dst = u32x2{lo, up};
      } else {
        *(uint32_t*)dst = lo;
      }
    }
  }

  // S^T[kb][qb] = K[32kb + sigma(.)] . Q[qb]^T for the 64-key tile in LDS.
  static __device__ __forceinline__ void qk(f32x16 (&s)[2][2], const Q& q, const uint16_t* sk,
                                            int col, int h) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 a = *(const bf16x8*)(sk + k_off(32 * kb + sigma(col), 2 * ks + h));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.r[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }
  }

  // O^T[db][qb] += V^T[db] P^T[qb]; P is the softmax numerator held in s.
  static __device__ __forceinline__ void pv(f32x16 (&o)[DB][2], const f32x16 (&s)[2][2],
                                            const uint16_t* svt, int col, int h) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 pb[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[qb][e] = (__bf16)s[kb][qb][8 * t + e];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          bf16x8 a = *(const bf16x8*)(svt + vt_off(db * 32 + col, 32 * kb + 16 * t + 8 * h));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], o[db][qb], 0, 0, 0);
        }
      }
    }
  }
};

// float inputs, v_mfma_f32_32x32x2_f32 (no reduced-precision step anywhere).
template <int D>
struct TraitsF32 {
  typedef float Elem;
  typedef float LA;
  typedef float LB;
  static constexpr int CPR = D / 4;                     // 16-byte chunks per row
  static constexpr int KCH = kKeysPerTile * CPR / 256;  // chunks per thread per tile (K and V)
  static constexpr int KS = D / 2;                      // QK k-steps
  static constexpr int DB = D / 32;
  static constexpr int STRIDE = D + 1;                  // padded LDS row (floats)
  static constexpr int A_ELEMS = kKeysPerTile * STRIDE;  // K stage
  static constexpr int B_ELEMS = kKeysPerTile * STRIDE;  // V stage

  struct Regs {
    f32x4 k[KCH];
    f32x4 v[KCH];
  };
  struct Q {
    float r[2][KS];
  };

  static __device__ __forceinline__ void load_q(Q& q, const void* qbase, int row0, int n_q,
                                                int col, int h) {
    const float* Qp = (const float*)qbase;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      int r = row0 + qb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) q.r[qb][ks] = r < n_q ? Qp[(size_t)r * D + 2 * ks + h] : 0.f;
    }
  }

  static __device__ __forceinline__ void load_tile(Regs& g, const void* kbase, const void* vbase,
                                                   int j0, int n_k, int tid) {
    const float* Kp = (const float*)kbase;
    const float* Vp = (const float*)vbase;
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int c = tid + 256 * p;
      int key = c / CPR, dc = c % CPR;
      int gk = j0 + key;
      g.k[p] = gk < n_k ? *(const f32x4*)(Kp + (size_t)gk * D + dc * 4) : f32x4{0, 0, 0, 0};
      g.v[p] = gk < n_k ? *(const f32x4*)(Vp + (size_t)gk * D + dc * 4) : f32x4{0, 0, 0, 0};
    }
  }

  static __device__ __forceinline__ void store_tile(const Regs& g, float* sk, float* sv, int tid) {
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int c = tid + 256 * p;
      int key = c / CPR, dc = c % CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[key * STRIDE + dc * 4 + e] = g.k[p][e];
        sv[key * STRIDE + dc * 4 + e] = g.v[p][e];
      }
    }
  }

  static __device__ __forceinline__ void qk(f32x16 (&s)[2][2], const Q& q, const float* sk,
                                            int col, int h) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float a = sk[(32 * kb + sigma(col)) * STRIDE + 2 * ks + h];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, q.r[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }
  }

  // Accumulator register u of block kb holds key 32kb + 16(u/8) + 8h + u%8.
  static __device__ __forceinline__ void pv(f32x16 (&o)[DB][2], const f32x16 (&s)[2][2],
                                            const float* sv, int col, int h) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        int key = 32 * kb + 16 * (u >> 3) + 8 * h + (u & 7);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float a = sv[key * STRIDE + db * 32 + col];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][qb][u], o[db][qb], 0, 0, 0);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// The step kernel.
// ---------------------------------------------------------------------------
template <typename Tr, int D, bool READ, bool FINAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void step_kernel(const StepArgs a) {
  typedef typename Tr::Elem E;
  typedef typename Tr::LA LA;
  typedef typename Tr::LB LB;
  constexpr int AE = Tr::A_ELEMS;
  constexpr int BE = Tr::B_ELEMS;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) LA s_a[2][AE];
  __shared__ __attribute__((aligned(16))) LB s_b[2][BE];
  __shared__ __attribute__((aligned(16))) int32_t s_pos[2][kKeysPerTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  const int u = blockIdx.x;
  const int head = a.head_of[u % a.h_q];
  const int qt = a.n_qt - 1 - u / a.h_q;
  const int kvh = head / (a.h_q / a.h_kv);
  const int row0_wg = qt * kRowsPerGroup;
  const int row0 = row0_wg + wave * kRowsPerWave;
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;

  // Key tiles this workgroup must visit: those whose first key is visible to
  // the group's last row (a prefix, since positions increase).
  const int n_kt = (n_k + kKeysPerTile - 1) / kKeysPerTile;
  const int wg_last = min(row0_wg + kRowsPerGroup, n_q) - 1;
  int n_iter = n_kt;
  if (causal) {
    const int qmax_wg = a.q_pos[wg_last];
    int cnt = 0;
    for (int j = lane; j < n_kt; j += 64) cnt += (a.k_pos[j * kKeysPerTile] <= qmax_wg) ? 1 : 0;
    n_iter = wave_sum_i(cnt);
  }

  const bool wave_valid = row0 < n_q;
  const bool count = a.work != nullptr && head == 0 && wave_valid;
  if (READ && !FINAL && n_iter == 0) {
    // No row of this group sees the block: the state stays as it is.
    if (count && lane == 0) atomicAdd(a.work + 2, (unsigned long long)n_kt);
    return;
  }

  // This wave's rows: extreme positions for tile classification and each
  // lane's own query position per 32-row block.
  const int wlast = min(row0 + kRowsPerWave, n_q) - 1;
  int qmin_w, qmax_w;
  if (!wave_valid) {
    qmin_w = kPosRowNone;
    qmax_w = kPosRowNone;
  } else if (causal) {
    qmin_w = a.q_pos[row0];
    qmax_w = a.q_pos[wlast];
  } else {
    qmin_w = kPosRowAll;
    qmax_w = kPosRowAll;
  }
  int qp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int r = row0 + qb * 32 + col;
    qp[qb] = r < n_q ? (causal ? a.q_pos[r] : kPosRowAll) : kPosRowNone;
  }

  const size_t qoff = ((size_t)head * n_q) * D;
  const size_t kvoff = ((size_t)kvh * n_k) * D;
  typename Tr::Q q;
  Tr::load_q(q, (const E*)a.q + qoff, row0, n_q, col, h);
  const E* kbase = (const E*)a.k + kvoff;
  const E* vbase = (const E*)a.v + kvoff;

  // Running state in base-2 units: m2 = max(scale*log2e * s); lsum = this
  // half-wave's share of the exp-sum; o = O^T accumulators.
  // m_nat0 / m2_0 remember the state's max as read, so a row whose max does
  // not move writes back the identical bits (no ln2 round trip).
  f32x16 o[DB][2];
  float m2[2], lsum[2], m_nat0[2], m2_0[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m2[qb] = -INFINITY;
    m_nat0[qb] = -INFINITY;
    lsum[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db][qb] = f32x16{};
  }
  if (READ) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      int r = row0 + qb * 32 + col;
      if (r < n_q) {
        size_t sr = (size_t)head * n_q + r;
        float mn = a.m_in[sr];
        m_nat0[qb] = mn;
        m2[qb] = mn * kLog2e;  // -inf stays -inf
        lsum[qb] = h == 0 ? a.l_in[sr] : 0.f;
        const float* orow = a.o_in + sr * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 x = *(const f32x4*)(orow + db * 32 + 8 * g + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[db][qb][4 * g + e] = x[e];
          }
      }
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) m2_0[qb] = m2[qb];

  int cnt_full = 0, cnt_masked = 0;
  const float c2 = a.c2;

  typename Tr::Regs g;
  if (n_iter > 0) {
    Tr::load_tile(g, kbase, vbase, 0, n_k, tid);
    if (tid < kKeysPerTile) {
      int gk = tid;
      s_pos[0][tid] = gk < n_k ? (causal ? a.k_pos[gk] : kPosAlways) : kPosHidden;
    }
    Tr::store_tile(g, s_a[0], s_b[0], tid);
  }
  __syncthreads();

  for (int j = 0; j < n_iter; ++j) {
    const int st = j & 1;
    const bool more = j + 1 < n_iter;
    int next_pos = kPosHidden;
    if (more) {
      const int j1 = (j + 1) * kKeysPerTile;
      Tr::load_tile(g, kbase, vbase, j1, n_k, tid);
      if (tid < kKeysPerTile) {
        int gk = j1 + tid;
        next_pos = gk < n_k ? (causal ? a.k_pos[gk] : kPosAlways) : kPosHidden;
      }
    }

    // Classify this tile for this wave's rows (valid keys only).
    const int j0 = j * kKeysPerTile;
    const int last_valid = min(j0 + kKeysPerTile, n_k) - 1 - j0;
    const int kmin = s_pos[st][0];
    const int kmax = s_pos[st][last_valid];
    const bool ragged = j0 + kKeysPerTile > n_k;
    const bool skip = !wave_valid || kmin > qmax_w;
    const bool full = kmax <= qmin_w;

    if (!skip) {
      if (full) ++cnt_full; else ++cnt_masked;
      f32x16 s[2][2];
      Tr::qk(s, q, s_a[st], col, h);
      if (!full || ragged) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          i32x4 kp4[4];
#pragma unroll
          for (int x = 0; x < 4; ++x)
            kp4[x] = *(const i32x4*)&s_pos[st][32 * kb + 8 * h + 16 * (x >> 1) + 4 * (x & 1)];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int kp = kp4[r >> 2][r & 3];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              s[kb][qb][r] = (kp <= qp[qb]) ? s[kb][qb][r] : -INFINITY;
          }
        }
      }
      // Online softmax: new max, rescale old totals, exponentiate.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = half_swap_max(mx);
        const float mnew = fmaxf(m2[qb], mx * c2);
        const float alpha = (m2[qb] == -INFINITY) ? 0.f : fast_exp2(m2[qb] - mnew);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(__builtin_fmaf(s[kb][qb][r], c2, -muse));
            s[kb][qb][r] = p;
            ps += p;
          }
        lsum[qb] = lsum[qb] * alpha + ps;
        m2[qb] = mnew;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db][qb] *= alpha;
      }
      Tr::pv(o, s, s_b[st], col, h);
    }

    if (more) {
      Tr::store_tile(g, s_a[st ^ 1], s_b[st ^ 1], tid);
      if (tid < kKeysPerTile) s_pos[st ^ 1][tid] = next_pos;
    }
    __syncthreads();
  }

  if (count && lane == 0) {
    atomicAdd(a.work + 0, (unsigned long long)cnt_full);
    atomicAdd(a.work + 1, (unsigned long long)cnt_masked);
    atomicAdd(a.work + 2, (unsigned long long)(n_kt - cnt_full - cnt_masked));
  }

  // Epilogue: combine the half-wave sums and write the state or the result.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ltot = half_swap_sum(lsum[qb]);
    const float m_nat = (m2[qb] == m2_0[qb]) ? m_nat0[qb] : m2[qb] * kLn2;
    const int r = row0 + qb * 32 + col;
    if (r >= n_q) continue;
    const size_t sr = (size_t)head * n_q + r;
    if (FINAL) {
      const bool ok = ltot > 0.f;
      const float inv = ok ? 1.f / ltot : 0.f;
      float* orow = a.out + sr * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = o[db][qb][4 * gq + e] * inv;
          *(f32x4*)(orow + db * 32 + 8 * gq + 4 * h) = x;
        }
      if (h == 0) a.lse[sr] = ok ? m_nat + logf(ltot) : -INFINITY;
    } else {
      float* orow = a.o_out + sr * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = o[db][qb][4 * gq + e];
          *(f32x4*)(orow + db * 32 + 8 * gq + 4 * h) = x;
        }
      if (h == 0) {
        a.m_out[sr] = m_nat;
        a.l_out[sr] = ltot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small kernels: state init, finalize, zero counters.
// ---------------------------------------------------------------------------
__global__ void state_init_kernel(float* m, float* l, float* o, int64_t rows, int d_k) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t n4 = rows * d_k / 4;
  if (i < n4) ((f32x4*)o)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (i < rows) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
}

__global__ void finalize_kernel(const float* m, const float* l, const float* o, float* out,
                                float* lse, int64_t rows, int d_k) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int per_row = d_k / 4;
  int64_t n4 = rows * per_row;
  if (i >= n4) return;
  int64_t r = i / per_row;
  float lv = l[r];
  bool ok = lv > 0.f;
  float inv = ok ? 1.f / lv : 0.f;
  f32x4 x = ((const f32x4*)o)[i];
  ((f32x4*)out)[i] = x * inv;
  if (i % per_row == 0) lse[r] = ok ? m[r] + logf(lv) : -INFINITY;
}

__global__ void zero_i64_kernel(int64_t* p, int n) {
  int i = threadIdx.x;
  if (i < n) p[i] = 0;
}

template <typename Tr, int D>
static hipError_t launch_typed(const StepArgs& a, bool read, bool final_, hipStream_t stream) {
  dim3 grid((unsigned)(a.n_qt * a.h_q)), block(256);
  if (read && final_)
    hipLaunchKernelGGL((step_kernel<Tr, D, true, true>), grid, block, 0, stream, a);
  else if (read)
    hipLaunchKernelGGL((step_kernel<Tr, D, true, false>), grid, block, 0, stream, a);
  else if (final_)
    hipLaunchKernelGGL((step_kernel<Tr, D, false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((step_kernel<Tr, D, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, int dtype, int d_k, bool read, bool final_,
                       hipStream_t stream) {
  if (dtype == 0) {
    if (d_k == 128) return launch_typed<TraitsBf16<128>, 128>(a, read, final_, stream);
    return launch_typed<TraitsBf16<64>, 64>(a, read, final_, stream);
  }
  if (d_k == 128) return launch_typed<TraitsF32<128>, 128>(a, read, final_, stream);
  return launch_typed<TraitsF32<64>, 64>(a, read, final_, stream);
}

hipError_t launch_state_init(float* m, float* l, float* o, int64_t rows, int d_k,
                             hipStream_t stream) {
  int64_t n = rows * d_k / 4;
  if (rows > n) n = rows;
  if (n == 0) return hipSuccess;
  unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(state_init_kernel, dim3(blocks), dim3(256), 0, stream, m, l, o, rows, d_k);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* m, const float* l, const float* o, float* out, float* lse,
                           int64_t rows, int d_k, hipStream_t stream) {
  int64_t n = rows * d_k / 4;
  if (n == 0) return hipSuccess;
  unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(finalize_kernel, dim3(blocks), dim3(256), 0, stream, m, l, o, out, lse, rows,
                     d_k);
  return hipGetLastError();
}

hipError_t launch_zero_i64(int64_t* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i64_kernel, dim3(1), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace ra
