// HIP kernels for one ring step of causal attention on gfx950 (MI355X).
//
// What a step computes (Zero to Frontier, "distributed/context-expert",
// section "Splitting the sequence, and the one layer that objects"): every
// local query meets one key/value block; its running maximum, running sum of
// exponentials and running weighted sum of values are rescaled when the block
// brings a larger score, then the block's terms are added.  Done one 64-key
// tile at a time inside the block, this is the blockwise online softmax the
// "Context Parallelism (CP)" concept page names in "Key math / How it works".
//
// Mapping onto CDNA4:
//  * A workgroup is 4 waves (one per SIMD) and owns a pair of 128-row query
//    tiles of one head (tile t and its mirror n_qt-1-t, processed in turn, so
//    causal triangles and zigzag steps give every workgroup the same work).
//    Each wave owns 32 query rows and has the SIMD's whole register file, so
//    operands can be fetched from LDS well ahead of their MFMAs.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (fp32 inputs: v_mfma_f32_32x32x2_f32).  K is the A operand, read from
//    LDS; Q is the B operand and stays in registers.  In the S^T accumulator
//    every lane holds one query column and 16 keys, so row max and row sum are
//    in-lane, plus one v_permlane32_swap between the two half-waves.
//  * Accumulator rows map to keys through sigma (swap of index bits 2 and 3),
//    which makes a half-wave's 8 P values of a 16-key step 8 consecutive keys:
//    P^T then feeds the PV MFMA (O^T = V^T P^T) as the B operand straight from
//    the accumulators, and V^T staged in LDS gives the A operand in one
//    16-byte read.
//  * Software pipeline: while tile j's softmax runs on the VALU, the MFMA
//    pipe runs the PV of tile j-1 and the QK of tile j+1, neither of which
//    depends on it.  K tiles are staged two tiles ahead and V tiles one ahead
//    (register-staged 16-byte loads, padded LDS rows), so one barrier per
//    tile suffices.
//  * Rescale on demand: O and l are multiplied by exp(m_old - m_new) only on
//    tiles where some row of the wave raised its maximum (a wave-wide ballot);
//    once a row has seen a few hundred keys that is rare.  m stays the exact
//    running maximum, so the largest P of a row is exactly 1 and its bf16
//    rounding costs nothing (a slack that let P exceed 1 cost ~3x in output
//    error on peaky rows).
//  * Tiles are classified from the explicit positions: skipped (no visible
//    pair), full, or masked (diagonal or ragged).  Only masked tiles compare
//    positions.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {

#ifndef RA_SCHED_PREFETCH
#define RA_SCHED_PREFETCH 4
#endif
#ifndef RA_SCHED_VALU
#define RA_SCHED_VALU 4
#endif
#ifndef RA_BF16_WAVES_PER_EU
#define RA_BF16_WAVES_PER_EU 1
#endif

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
constexpr int kPosLoNone = (int)0x80000000;   // no lower bound on a row's visible keys

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
// Element-type traits.  Each provides the Q registers, staging of K / V tiles
// from HBM through registers into LDS, S^T = K Q^T for one 32-key half of a
// tile, the exponentials of one half (returning the PV operand and adding to
// the row sum), and O^T += V^T P^T for one half.
// ---------------------------------------------------------------------------

// bfloat16 inputs, v_mfma_f32_32x32x16_bf16.
template <int D>
struct TraitsBf16 {
  typedef uint16_t Elem;   // bfloat16 bits in HBM
  typedef uint16_t LK;     // LDS element of the K stage
  typedef uint16_t LV;     // LDS element of the V^T stage
  static constexpr int WAVES_PER_EU = RA_BF16_WAVES_PER_EU;
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int KCH = kKeysPerTile * CPR / 256;   // K chunks per thread per tile
  static constexpr int NV = KCH;                         // V keys per thread per tile
  static constexpr int KS = D / 16;                      // QK k-steps
  static constexpr int DB = D / 32;                      // 32-wide d blocks of O^T
  static constexpr int KSTR = D + 8;                     // padded K row (elements)
  static constexpr int VSTR = kKeysPerTile + 8;          // padded V^T row (elements)
  static constexpr int K_ELEMS = kKeysPerTile * KSTR;
  static constexpr int V_ELEMS = D * VSTR;

  struct KRegs { u32x4 c[KCH]; };
  struct VRegs { u32x4 c[NV]; };
  struct Q { bf16x8 r[KS]; };
  struct P { bf16x8 t[2]; };

  // Rows are padded by 16 bytes: 16 consecutive rows read at the same column
  // fall on 16 distinct groups of 4 banks, and every offset inside the tile
  // loops is a compile-time immediate.
  static __device__ __forceinline__ int k_off(int key, int chunk) { return key * KSTR + chunk * 8; }
  static __device__ __forceinline__ int vt_off(int d, int key) { return d * VSTR + key; }

  static __device__ __forceinline__ void load_q(Q& q, const Elem* qbase, int row, int n_q, int h) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      q.r[ks] = row < n_q ? *(const bf16x8*)(qbase + (size_t)row * D + ks * 16 + h * 8) : bf16x8{};
  }

  static __device__ __forceinline__ void load_k(KRegs& g, const Elem* kb, int j0, int n_k, int tid) {
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int c = tid + 256 * p;
      int key = c / CPR, dc = c % CPR;
      int gk = j0 + key;
      // Rows past the block are read from its last row and zeroed, so the
      // load needs no branch.
      u32x4 x = *(const u32x4*)(kb + (size_t)min(gk, n_k - 1) * D + dc * 8);
      g.c[p] = gk < n_k ? x : u32x4{0, 0, 0, 0};
    }
  }
  static __device__ __forceinline__ void store_k(const KRegs& g, LK* sk, int tid) {
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int c = tid + 256 * p;
      int key = c / CPR, dc = c % CPR;
      *(u32x4*)(sk + k_off(key, dc)) = g.c[p];
    }
  }
  // Each thread loads NV consecutive keys x 8 d values and writes them
  // transposed into V^T rows 8*dc .. 8*dc+7.  Lanes of one store cover
  // consecutive keys of one row, so the stores do not conflict.
  static __device__ __forceinline__ void load_v(VRegs& g, const Elem* vb, int j0, int n_k, int tid) {
    constexpr int KG = kKeysPerTile / NV;
    int kg = tid % KG, dc = tid / KG;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int gk = j0 + kg * NV + i;
      u32x4 x = *(const u32x4*)(vb + (size_t)min(gk, n_k - 1) * D + dc * 8);
      g.c[i] = gk < n_k ? x : u32x4{0, 0, 0, 0};
    }
  }
  static __device__ __forceinline__ void store_v(const VRegs& g, LV* svt, int tid) {
    constexpr int KG = kKeysPerTile / NV;
    int kg = tid % KG, dc = tid / KG;
    int key0 = kg * NV;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int w = e >> 1;
      bool hi = e & 1;
      int d = dc * 8 + e;
      uint32_t a0 = g.c[0][w], a1 = g.c[1][w];
      uint32_t lo = hi ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
      LV* dst = svt + vt_off(d, key0);
      if constexpr (NV == 4) {
        uint32_t a2 = g.c[2][w], a3 = g.c[3][w];
        uint32_t up = hi ? ((a2 >> 16) | (a3 & 0xffff0000u)) : ((a2 & 0xffffu) | (a3 << 16));
        *(u32x2*)dst = u32x2{lo, up};
      } else {
        *(uint32_t*)dst = lo;
      }
    }
  }

  // S^T rows 32kb..32kb+31 (keys 32kb + sigma(.)) against this wave's Q.
  static __device__ __forceinline__ f32x16 qk(const Q& q, const LK* sk, int kb, int col, int h) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 a = *(const bf16x8*)(sk + k_off(32 * kb + sigma(col), 2 * ks + h));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.r[ks], s, 0, 0, 0);
    }
    return s;
  }

  // P = 2^(s*c2 - m) rounded to bf16 for the PV product; the row sum adds
  // the fp32 values (summing the rounded values costs ~1e-3 in lse when one
  // key dominates a row).
  static __device__ __forceinline__ P exp_pack(const f32x16& s, float c2, float m, float& lsum) {
    P p;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float x0 = fast_exp2(__builtin_fmaf(s[8 * t + e], c2, -m));
        float x1 = fast_exp2(__builtin_fmaf(s[8 * t + e + 1], c2, -m));
        p.t[t][e] = (__bf16)x0;
        p.t[t][e + 1] = (__bf16)x1;
        acc0 += x0;
        acc1 += x1;
      }
    lsum += acc0 + acc1;
    return p;
  }

  // O^T[db] += V^T[db rows, keys 32kb + ...] P^T.
  static __device__ __forceinline__ void pv(f32x16 (&o)[DB], const P& p, const LV* svt, int kb,
                                            int col, int h) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8 a = *(const bf16x8*)(svt + vt_off(db * 32 + col, 32 * kb + 16 * t + 8 * h));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p.t[t], o[db], 0, 0, 0);
      }
  }
};

// float inputs, v_mfma_f32_32x32x2_f32 (no reduced-precision step anywhere).
template <int D>
struct TraitsF32 {
  typedef float Elem;
  typedef float LK;
  typedef float LV;
  static constexpr int WAVES_PER_EU = 1;
  static constexpr int CPR = D / 4;                     // 16-byte chunks per row
  static constexpr int KCH = kKeysPerTile * CPR / 256;  // chunks per thread per tile
  static constexpr int KS = D / 2;                      // QK k-steps
  static constexpr int DB = D / 32;
  static constexpr int STR = D + 1;                     // padded LDS row (floats)
  static constexpr int K_ELEMS = kKeysPerTile * STR;
  static constexpr int V_ELEMS = kKeysPerTile * STR;

  struct KRegs { f32x4 c[KCH]; };
  struct VRegs { f32x4 c[KCH]; };
  struct Q { float r[KS]; };
  struct P { f32x16 v; };

  static __device__ __forceinline__ void load_q(Q& q, const Elem* qbase, int row, int n_q, int h) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q.r[ks] = row < n_q ? qbase[(size_t)row * D + 2 * ks + h] : 0.f;
  }
  static __device__ __forceinline__ void load_rows(f32x4 (&c)[KCH], const Elem* base, int j0,
                                                   int n_k, int tid) {
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int ci = tid + 256 * p;
      int key = ci / CPR, dc = ci % CPR;
      int gk = j0 + key;
      f32x4 x = *(const f32x4*)(base + (size_t)min(gk, n_k - 1) * D + dc * 4);
      c[p] = gk < n_k ? x : f32x4{0, 0, 0, 0};
    }
  }
  static __device__ __forceinline__ void store_rows(const f32x4 (&c)[KCH], float* sm, int tid) {
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      int ci = tid + 256 * p;
      int key = ci / CPR, dc = ci % CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm[key * STR + dc * 4 + e] = c[p][e];
    }
  }
  static __device__ __forceinline__ void load_k(KRegs& g, const Elem* kb, int j0, int n_k, int tid) {
    load_rows(g.c, kb, j0, n_k, tid);
  }
  static __device__ __forceinline__ void store_k(const KRegs& g, LK* sk, int tid) {
    store_rows(g.c, sk, tid);
  }
  static __device__ __forceinline__ void load_v(VRegs& g, const Elem* vb, int j0, int n_k, int tid) {
    load_rows(g.c, vb, j0, n_k, tid);
  }
  static __device__ __forceinline__ void store_v(const VRegs& g, LV* sv, int tid) {
    store_rows(g.c, sv, tid);
  }

  static __device__ __forceinline__ f32x16 qk(const Q& q, const LK* sk, int kb, int col, int h) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float a = sk[(32 * kb + sigma(col)) * STR + 2 * ks + h];
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a, q.r[ks], s, 0, 0, 0);
    }
    return s;
  }

  static __device__ __forceinline__ P exp_pack(const f32x16& s, float c2, float m, float& lsum) {
    P p;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p.v[r] = fast_exp2(__builtin_fmaf(s[r], c2, -m));
      lsum += p.v[r];
    }
    return p;
  }

  // Accumulator register u holds key 32kb + 16(u/8) + 8h + u%8.
  static __device__ __forceinline__ void pv(f32x16 (&o)[DB], const P& p, const LV* sv, int kb,
                                            int col, int h) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      int key = 32 * kb + 16 * (u >> 3) + 8 * h + (u & 7);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float a = sv[key * STR + db * 32 + col];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p.v[u], o[db], 0, 0, 0);
      }
    }
  }
};

template <typename Tr>
struct Smem {
  typename Tr::LK k[2][Tr::K_ELEMS];
  typename Tr::LV v[2][Tr::V_ELEMS];
  int32_t pos[3][kKeysPerTile];
};

// Masks hidden keys of one 32-key half to -inf: those after the query (qp)
// and those before its lower bound (qlo, the document start).  Accumulator
// register r of half kb holds tile key 32kb + 8h + 16(r/8) + r%8.
__device__ __forceinline__ void apply_mask(f32x16& s, const int32_t* pos, int kb, int h, int qp,
                                           int qlo) {
  i32x4 kp4[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
    kp4[x] = *(const i32x4*)&pos[32 * kb + 8 * h + 16 * (x >> 1) + 4 * (x & 1)];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kp = kp4[r >> 2][r & 3];
    s[r] = (kp <= qp && kp >= qlo) ? s[r] : -INFINITY;
  }
}

// Position of key gk of the block as the tile masks see it (branch-free:
// the load is clamped into the block).  Requires n_k >= 1.
__device__ __forceinline__ int key_pos(const StepArgs& a, int gk, bool causal) {
  const int p = a.k_pos[min(gk, a.n_k - 1)];
  return gk < a.n_k ? (causal ? p : kPosAlways) : kPosHidden;
}

// One 128-row query tile of one head against the whole key/value block.
//
// Pipeline, per wave, for key tile j (PV(j-1) and QK(j+1) are independent of
// the softmax of tile j, so the MFMA and VALU streams of an iteration overlap):
//   MFMA: O^T += V_{j-1}^T P_{j-1}^T        (previous tile's probabilities)
//         S_{j+1}^T = K_{j+1} Q^T          (next tile's scores)
//   VALU: mask S_j (diagonal/ragged tiles), row max, P_j = 2^(S_j c - m)
//   O is rescaled, if the max moved, at the top of the next iteration (after
//   PV(j-1), before PV(j)).
// LDS: K_{j+1} and V_{j-1} are read while K_{j+2} and V_j are written to the
// other stages, so one barrier per tile orders everything.
template <typename Tr, int D, bool READ, bool FINAL>
struct QTile {
  typedef typename Tr::Elem E;
  static constexpr int DB = D / 32;

  const StepArgs& a;
  Smem<Tr>& sm;
  const int tid, lane, wave, h, col;
  const int n_q, n_k;
  const bool causal;
  const E* kbase;
  const E* vbase;
  int n_iter = 0;
  bool wave_valid = false;
  int qmin_w = 0, qmax_w = 0, qp = 0;
  // Lower bounds of the visible key positions: this lane's row, and the
  // smallest and largest over the wave's rows (kPosLoNone without a bound).
  int qlo = kPosLoNone, qlo_min_w = kPosLoNone, qlo_max_w = kPosLoNone;
  float c2 = 0.f;

  typename Tr::Q q;
  f32x16 o[DB];
  float m2 = -INFINITY, lsum = 0.f;
  int cnt_full = 0, cnt_masked = 0;
  typename Tr::KRegs gk;
  typename Tr::VRegs gv;
  f32x16 s_cur[2], s_next[2];
  typename Tr::P p_prev[2];
  bool need_rescale = false;
  float alpha_pending = 1.f;

  __device__ QTile(const StepArgs& a_, Smem<Tr>& sm_, int tid_)
      : a(a_), sm(sm_), tid(tid_), lane(tid_ & 63),
        wave(__builtin_amdgcn_readfirstlane(tid_ >> 6)), h((tid_ & 63) >> 5),
        col(tid_ & 31), n_q(a_.n_q), n_k(a_.n_k), causal(a_.causal != 0), kbase(nullptr),
        vbase(nullptr) {}

  // Scheduling hint for the iteration's main block: alternate one MFMA, one
  // LDS read and a few VALU instructions, with a few LDS reads issued ahead,
  // so the softmax fills the MFMA pipe's shadow and operand reads are in
  // flight before their MFMAs.
  template <int NM>
  __device__ __forceinline__ static void interleave() {
    if constexpr (NM > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, RA_SCHED_PREFETCH, 0);  // DS read
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);               // DS read
        __builtin_amdgcn_sched_group_barrier(0x402, RA_SCHED_VALU, 0);   // VALU incl. exp
      }
    }
  }

  // Rescale O when the previous iteration's softmax moved the max.  It runs
  // at the top of an iteration: after PV(j-2) (issued last iteration) and
  // before PV(j-1), and outside the block where MFMAs and exponentials
  // interleave.
  __device__ __forceinline__ void apply_pending_rescale() {
    if (need_rescale) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha_pending;
    }
  }

  template <bool PV_PREV, bool QK_NEXT>
  __device__ __forceinline__ void iteration(int j) {
    apply_pending_rescale();
    // Staging loads: K two tiles ahead (clamped; a repeated tile lands in a
    // stage nobody reads), V of this tile for the next iteration's PV.
    const int jk = min(j + 2, n_iter - 1);
    Tr::load_k(gk, kbase, jk * kKeysPerTile, n_k, tid);
    // Every thread fetches one position; the four waves write the same 64
    // values, which keeps the block free of divergent branches.
    const int next_pos = key_pos(a, jk * kKeysPerTile + (tid & (kKeysPerTile - 1)), causal);
    Tr::load_v(gv, vbase, j * kKeysPerTile, n_k, tid);

    // Classify tile j for this wave's rows (valid keys only).
    const int32_t* pos = sm.pos[j % 3];
    const int j0 = j * kKeysPerTile;
    const int last_valid = min(j0 + kKeysPerTile, n_k) - 1 - j0;
    const int kmin = pos[0], kmax = pos[last_valid];
    const bool ragged = j0 + kKeysPerTile > n_k;
    const bool skip = !wave_valid || kmin > qmax_w || kmax < qlo_min_w;
    const bool full = kmax <= qmin_w && kmin >= qlo_max_w;
    if (!skip) {
      if (full) ++cnt_full; else ++cnt_masked;
    }
    if (skip || !full || ragged) {
      // A skipped tile is masked completely: P = 0, nothing changes.
      const int qpe = skip ? kPosRowNone : qp;
      apply_mask(s_cur[0], pos, 0, h, qpe, qlo);
      apply_mask(s_cur[1], pos, 1, h, qpe, qlo);
    }

    // ---- one branch-free block: MFMA stream and softmax interleave ----
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s_cur[0][r], s_cur[1][r]));
    const float mloc = half_swap_max(mx) * c2;
    need_rescale = __ballot(mloc > m2) != 0;
    const float mnew = fmaxf(m2, mloc);
    alpha_pending = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mnew);
    m2 = mnew;
    // A row with nothing visible yet keeps m2 = -inf and gets P = 0.
    const float muse = (m2 == -INFINITY) ? 0.f : m2;

    if (PV_PREV) {
      Tr::pv(o, p_prev[0], sm.v[(j - 1) & 1], 0, col, h);
      Tr::pv(o, p_prev[1], sm.v[(j - 1) & 1], 1, col, h);
    }
    if (QK_NEXT) {
      s_next[0] = Tr::qk(q, sm.k[(j + 1) & 1], 0, col, h);
      s_next[1] = Tr::qk(q, sm.k[(j + 1) & 1], 1, col, h);
    }
    lsum *= alpha_pending;
    p_prev[0] = Tr::exp_pack(s_cur[0], c2, muse, lsum);
    p_prev[1] = Tr::exp_pack(s_cur[1], c2, muse, lsum);

    Tr::store_k(gk, sm.k[j & 1], tid);
    sm.pos[(j + 2) % 3][tid & (kKeysPerTile - 1)] = next_pos;
    Tr::store_v(gv, sm.v[j & 1], tid);
    interleave<(PV_PREV ? 16 : 0) + (QK_NEXT ? 16 : 0)>();
    __syncthreads();
    if (QK_NEXT) {
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
    }
  }

  __device__ void run(int qt, int head) {
    const int kvh = head / (a.h_q / a.h_kv);
    const int row0_wg = qt * kRowsPerGroup;
    const int row0 = row0_wg + wave * kRowsPerWave;

    // Key tiles this workgroup visits: those whose first key is visible to
    // the group's last row (a prefix, since positions increase).
    const int n_kt = (n_k + kKeysPerTile - 1) / kKeysPerTile;
    n_iter = n_kt;
    if (causal) {
      const int qmax_wg = a.q_pos[min(row0_wg + kRowsPerGroup, n_q) - 1];
      int cnt = 0;
      for (int j = lane; j < n_kt; j += 64) cnt += (a.k_pos[j * kKeysPerTile] <= qmax_wg) ? 1 : 0;
      n_iter = wave_sum_i(cnt);
    }
    wave_valid = row0 < n_q;
    const bool count = a.work != nullptr && head == 0 && wave_valid;
    if (READ && !FINAL && n_iter == 0) {
      // No row of this tile sees the block: its state stays as it is.
      if (count && lane == 0) atomicAdd(a.work + 2, (unsigned long long)n_kt);
      return;
    }

    // This wave's rows and this lane's query position.
    if (!wave_valid) {
      qmin_w = qmax_w = kPosRowNone;
    } else if (causal) {
      qmin_w = a.q_pos[row0];
      qmax_w = a.q_pos[min(row0 + kRowsPerWave, n_q) - 1];
    } else {
      qmin_w = qmax_w = kPosRowAll;
    }
    const int row = row0 + col;
    qp = row < n_q ? (causal ? a.q_pos[row] : kPosRowAll) : kPosRowNone;
    if (a.q_lo != nullptr && wave_valid) {
      // Lower bounds never decrease along the rows (documents follow the
      // positions), so the wave's first and last rows give its extremes.
      qlo_min_w = a.q_lo[row0];
      qlo_max_w = a.q_lo[min(row0 + kRowsPerWave, n_q) - 1];
      qlo = row < n_q ? a.q_lo[row] : kPosLoNone;
    }

    kbase = (const E*)a.k + ((size_t)kvh * n_k) * D;
    vbase = (const E*)a.v + ((size_t)kvh * n_k) * D;
    Tr::load_q(q, (const E*)a.q + ((size_t)head * n_q) * D, row, n_q, h);

    // Running state in base-2 units: m2 is the running maximum the sums are
    // taken against, lsum this half-wave's share of the exp-sum, o the O^T
    // accumulators.  m_nat0 / m2_0 keep the state's max as read, so a row
    // whose max does not move writes back the identical bits.
    float m_nat0 = -INFINITY;
    m2 = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    const size_t srow = (size_t)head * n_q + row;
    if (READ && row < n_q) {
      m_nat0 = a.m_in[srow];
      m2 = m_nat0 * kLog2e;  // -inf stays -inf
      lsum = h == 0 ? a.l_in[srow] : 0.f;
      const float* orow = a.o_in + srow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x = *(const f32x4*)(orow + db * 32 + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][4 * g + e] = x[e];
        }
    }
    const float m2_0 = m2;
    c2 = a.c2;
    cnt_full = cnt_masked = 0;
    need_rescale = false;

    if (n_iter > 0) {
      // Prologue: K0, K1 and their positions into LDS, then S^T of tile 0.
      Tr::load_k(gk, kbase, 0, n_k, tid);
      if (tid < kKeysPerTile) sm.pos[0][tid] = key_pos(a, tid, causal);
      Tr::store_k(gk, sm.k[0], tid);
      if (n_iter > 1) {
        Tr::load_k(gk, kbase, kKeysPerTile, n_k, tid);
        if (tid < kKeysPerTile) sm.pos[1][tid] = key_pos(a, kKeysPerTile + tid, causal);
        Tr::store_k(gk, sm.k[1], tid);
      }
      __syncthreads();
      s_cur[0] = Tr::qk(q, sm.k[0], 0, col, h);
      s_cur[1] = Tr::qk(q, sm.k[0], 1, col, h);
      __syncthreads();  // K stage 0 is refilled during the first iteration

      if (n_iter == 1) {
        iteration<false, false>(0);
      } else {
        iteration<false, true>(0);
        for (int j = 1; j < n_iter - 1; ++j) iteration<true, true>(j);
        iteration<true, false>(n_iter - 1);
      }
      // The last tile's PV.
      apply_pending_rescale();
      Tr::pv(o, p_prev[0], sm.v[(n_iter - 1) & 1], 0, col, h);
      Tr::pv(o, p_prev[1], sm.v[(n_iter - 1) & 1], 1, col, h);
    }

    if (count && lane == 0) {
      atomicAdd(a.work + 0, (unsigned long long)cnt_full);
      atomicAdd(a.work + 1, (unsigned long long)cnt_masked);
      atomicAdd(a.work + 2, (unsigned long long)(n_kt - cnt_full - cnt_masked));
    }

    // Epilogue: combine the half-wave sums and write the state or the result.
    const float ltot = half_swap_sum(lsum);
    if (row >= n_q) return;
    const float m_nat = (m2 == m2_0) ? m_nat0 : m2 * kLn2;
    if (FINAL) {
      const bool ok = ltot > 0.f;
      const float inv = ok ? 1.f / ltot : 0.f;
      float* orow = a.out + srow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = o[db][4 * g + e] * inv;
          *(f32x4*)(orow + db * 32 + 8 * g + 4 * h) = x;
        }
      if (h == 0) a.lse[srow] = ok ? m_nat + logf(ltot) : -INFINITY;
    } else {
      float* orow = a.o_out + srow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = o[db][4 * g + e];
          *(f32x4*)(orow + db * 32 + 8 * g + 4 * h) = x;
        }
      if (h == 0) {
        a.m_out[srow] = m_nat;
        a.l_out[srow] = ltot;
      }
    }
  }
};

// One workgroup: a query head and a pair of query tiles (heavier one first).
template <typename Tr, int D, bool READ, bool FINAL>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(Tr::WAVES_PER_EU, Tr::WAVES_PER_EU)))
void step_kernel(const StepArgs a) {
  __shared__ __attribute__((aligned(16))) Smem<Tr> sm;
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int head = a.head_of[u % a.h_q];
  const int p = u / a.h_q;
  const int t_hi = a.n_qt - 1 - p, t_lo = p;
  QTile<Tr, D, READ, FINAL> t(a, sm, tid);
  t.run(t_hi, head);
  if (t_lo < t_hi) {
    __syncthreads();  // LDS of the first tile is fully consumed
    t.run(t_lo, head);
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

// Fills n floats with zero (a kernel, not a memset, so that a captured graph
// holds no memset node).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <typename Tr, int D>
static hipError_t launch_typed(const StepArgs& a, bool read, bool final_, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop) {
  dim3 grid((unsigned)(a.n_pairs * a.h_q)), block(256);
  auto go = [&](auto kernel) {
    if (start || stop)
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, a);
    else
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, a);
  };
  if (read && final_)
    go(step_kernel<Tr, D, true, true>);
  else if (read)
    go(step_kernel<Tr, D, true, false>);
  else if (final_)
    go(step_kernel<Tr, D, false, true>);
  else
    go(step_kernel<Tr, D, false, false>);
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, int dtype, int d_k, bool read, bool final_,
                       hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (dtype == 0) {
    if (d_k == 128) return launch_step_fast(a, read, final_, stream, start, stop);
    return launch_typed<TraitsBf16<64>, 64>(a, read, final_, stream, start, stop);
  }
  if (d_k == 128) return launch_typed<TraitsF32<128>, 128>(a, read, final_, stream, start, stop);
  return launch_typed<TraitsF32<64>, 64>(a, read, final_, stream, start, stop);
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

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p,
                     n);
  return hipGetLastError();
}

}  // namespace ra
