// Fast ring-step kernel for bfloat16 inputs with d_k = 128 on gfx950.
//
// Computes exactly what the generic step kernel computes (one key/value block
// folded into the online-softmax state, Zero to Frontier
// "distributed/context-expert", section "Splitting the sequence, and the one
// layer that objects"), organised for CDNA4 throughput:
//
//  * Two waves per SIMD, in one of two forms chosen per launch.  With fewer
//    than two workgroup-sized work units (query tile pair x head) per
//    compute unit, a workgroup is 8 waves: two groups of 4 waves on the same
//    128 query rows (32 per wave).  Group g takes the key tiles j = g, g+2,
//    g+4, ... of the block; the two partial states are folded together
//    through LDS at the end (the same online-softmax fold).  With at least
//    two units per compute unit, a workgroup is one group of 4 waves taking
//    every key tile, and two such workgroups share a compute unit: their
//    waves pair up on each SIMD without the barriers that tie the two
//    groups of one workgroup together (4-5% faster where it applies).
//  * No staging registers.  K and V tiles go from HBM straight into LDS with
//    buffer_load_dwordx4 ... lds, in row-major 256-byte rows whose 16-byte chunks
//    are XOR-swizzled by row, so both read patterns below are free of bank
//    conflicts.  That leaves each wave under 256 registers.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows are the A operand
//    (one ds_read_b128 each), Q stays in registers as the B operand.  Every
//    lane then holds one query column, so row max and row sum are in-lane
//    plus one v_permlane32_swap.  Accumulator row i holds key sigma(i) (index
//    bits 2 and 3 swapped), so P^T feeds O^T = V^T P^T straight from the
//    accumulators, 8 consecutive keys per half-wave.
//  * The V^T operand comes from row-major V with ds_read_b64_tr_b16: within
//    each 16-lane group, lane j receives element j of the 4 rows the group
//    addressed, i.e. 4 consecutive keys of one d column.
//  * Each group alternates a softmax phase (VALU: classify, mask, row max,
//    rescale, exponentials) and a GEMM phase (MFMA: P V of that tile, then
//    S^T of its next tile), with a workgroup barrier after every phase.  In
//    the two-group form group 1 runs one phase behind group 0 (a ping-pong),
//    so on each SIMD one wave keeps the matrix pipe busy while the other runs
//    the softmax, and every barrier swaps the roles.
//  * Loads are DMA issued three phases before their use and waited for with
//    explicit vmcnt counts; K and V tiles have two stages per group,
//    positions three.
//  * The all-gather form runs the same machinery over every resident block
//    in one launch, the state staying in registers.  Its document-mask
//    variant (DOCS) also bounds each query's keys below by its document
//    start; without it that code compiles away.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {
namespace fast {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int BN = 64;                      // keys per tile
constexpr int ROWS = 128;                   // query rows per workgroup tile
constexpr int WAVE_ROWS = 32;
// G, the groups of 4 waves in a workgroup, is a template parameter: 2 runs
// the ping-pong of the two groups on the same query rows, 1 a single group
// per workgroup with two workgroups resident per compute unit.
template <int G>
constexpr int threads() { return 256 * G; }
constexpr int TILE_BYTES = BN * D * 2;      // 16 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPosRowNone = (int)0x80000000;
constexpr int kPosRowAll = 0x7ffffffe;
constexpr int kPosLoNone = (int)0x80000000;  // no lower bound on a row's visible keys
// Word 3 of a raw (untyped, stride-0) buffer resource on gfx9: 32-bit data
// format; offsets at or past num_records read as zero.
constexpr int kBufferFlags = 0x00020000;

static_assert(ROWS == 4 * WAVE_ROWS, "4 waves per group");
static_assert(kRowsPerGroup == ROWS, "host launch geometry");

template <int G>
struct __attribute__((aligned(1024))) Smem {
  uint8_t k[G][2][TILE_BYTES];   // [group][stage]
  uint8_t v[G][2][TILE_BYTES];
  int32_t pos[G][3][BN];         // [group][stage]
};
// The merge of the two groups reuses the K/V area.
static_assert(4 * 64 * 64 * 4 + 4 * 64 * 2 * 4 <= (int)sizeof(uint8_t[2][2][TILE_BYTES]) * 2,
              "merge buffer fits");
// One group per workgroup: two workgroups fit the compute unit's 160 KiB.
static_assert(2 * sizeof(Smem<1>) <= 160 * 1024, "two one-group workgroups per CU");

// A value the compiler cannot see through.  With one group the group index
// is always 0; folding that constant into the loop bodies made the compiler
// hoist enough to spill 50-190 registers, so it is computed at run time.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

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

// Raw buffer resource (gfx9 layout): 48-bit base, stride 0, size in bytes,
// 32-bit untyped data; every word is wave-uniform.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int bytes) {
  const uint64_t b = (uint64_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xffff),
               __builtin_amdgcn_readfirstlane(bytes), kBufferFlags};
}

// Four 16-byte-per-lane buffer loads from HBM straight into LDS (4 KiB):
// load i of lane L reads global byte soff + 1024 i + voff_i and lands at LDS
// byte lds + 1024 i + 16 L (the instruction offset moves both addresses).
// Bytes at or past the resource size read as zero.  Issued as inline asm so
// the compiler does not track them: it cannot tell that the stage being
// filled is not the one being read, and would otherwise wait for the load
// before the very next LDS read.  Callers wait (vmcnt) before the barrier
// that publishes the stage.  M0 carries the LDS address; the nop is the
// required wait state between writing M0 and the LDS-DMA that reads it.
__device__ __forceinline__ void dma_tile_to_lds(const i32x4& rsrc, uint32_t lds, int v0, int v1,
                                                int v2, int v3, int soff) {
  const int m0v = __builtin_amdgcn_readfirstlane((int)lds);
  const int so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
      "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
      :
      : "s"(m0v), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(rsrc), "s"(so)
      : "m0");
}
// One 4-byte-per-lane load into LDS (lane L's word lands at lds + 4 L).
__device__ __forceinline__ void dma_words_to_lds(const i32x4& rsrc, uint32_t lds, int voff, int soff) {
  const int m0v = __builtin_amdgcn_readfirstlane((int)lds);
  const int so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc), "s"(so)
               : "m0");
}

// Byte offset of 16-byte chunk c of row r inside a K tile / a V tile.
__device__ __forceinline__ int k_chunk_off(int r, int c) { return r * 256 + 16 * (c ^ (r & 15)); }
__device__ __forceinline__ int v_chunk_off(int r, int c) { return r * 256 + 16 * (c ^ (4 * (r & 3))); }

template <int G, bool READ, bool FINAL, bool DOCS = false>
struct Step {
  const StepArgs& a;
  Smem<G>& sm;
  const int tid, lane, gwave, grp, h, col;
  const int n_q, n_k;
  const bool causal;
  const uint16_t* kbase;
  const uint16_t* vbase;
  int n_iter = 0, n_own = 0;
  bool wave_valid = false;
  int qmin_w = 0, qmax_w = 0, qp = 0;
  // Lower bounds of the visible key positions (document starts): this
  // lane's row, the wave's smallest and largest, the workgroup's smallest.
  int qlo = kPosLoNone, qlo_min_w = kPosLoNone, qlo_max_w = kPosLoNone, qlo_min_wg = kPosLoNone;
  // First key tile the workgroup visits in the current block (even, so each
  // group keeps its tile parity); 0 without lower bounds.
  int j0 = 0;
  int lo_vis_w = 0, lo_full_w = 0;  // this wave's first visible / fully visible tile
  // Without document masks all of this folds away to the plain causal case.
  __device__ __forceinline__ int tile0() const { return DOCS ? j0 : 0; }
  float c2 = 0.f;

  // Buffer resources of this head's K, V and key positions: loads past the
  // block's end return zeros, so ragged tiles need no clamping.
  i32x4 krs, vrs, prs;
  // per-lane offsets (loop invariant)
  uint32_t lds_k, lds_v, lds_pos;  // LDS byte addresses of this group's stages
  int k_ld_off[4];   // byte offset in a K tile of this lane's load i (relative to 1024 i)
  int v_ld_off;      // ditto for V (the same for every i)
  int k_rd;          // K read base, XOR'ed with 32*ks
  int v_rd;          // V read base, XOR'ed with 64*db

  bf16x8 q[8];
  f32x16 o[4];
  float m2 = -INFINITY, lsum = 0.f;
  int cnt_full = 0, cnt_masked = 0;
  int n_full_w = 0, n_vis_w = 0;  // key tiles this wave sees fully / at all
  bool resc = false;   // O must be scaled by alpha before the next PV
  float alpha = 1.f;
  f32x16 sc[2];        // scores of one own tile (S^T, two 32-key halves)
  bf16x8 pp[2][2];      // its probabilities, bf16

  __device__ Step(const StepArgs& a_, Smem<G>& sm_, int tid_)
      : a(a_), sm(sm_), tid(tid_), lane(tid_ & 63),
        gwave(__builtin_amdgcn_readfirstlane((tid_ >> 6) & 3)),
        grp(__builtin_amdgcn_readfirstlane(G == 1 ? opaque(tid_ >> 8) : tid_ >> 8)),
        h((tid_ & 63) >> 5), col(tid_ & 31),
        n_q(a_.n_q), n_k(a_.n_k), causal(a_.causal != 0), kbase(nullptr), vbase(nullptr) {
    // Tile loads: wave w fills rows 16w .. 16w+15 of a tile, load i rows
    // 16w + 4i + L/16 for lane L, which writes physical chunk L%16 of its
    // row: logical chunk (L%16) ^ (row & 15) for K, (L%16) ^ 4(row & 3) for V.
    {
      const int L = lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + L / 16;  // row within the wave's 16 (same & 15)
        k_ld_off[i] = (L / 16) * 256 + 16 * ((L % 16) ^ (r & 15));
      }
      v_ld_off = (L / 16) * 256 + 16 * ((L % 16) ^ (4 * ((L / 16) & 3)));
      const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)&sm_;
      lds_k = base + (uint32_t)offsetof(Smem<G>, k) + grp * 2 * TILE_BYTES;
      lds_v = base + (uint32_t)offsetof(Smem<G>, v) + grp * 2 * TILE_BYTES;
      lds_pos = base + (uint32_t)offsetof(Smem<G>, pos) + grp * 3 * BN * 4;
    }
    // K reads: row sigma(col) (+32 kb), logical chunk 2ks + h.
    {
      const int r = sigma(col);
      const int x = r & 15;
      k_rd = r * 256 + 16 * (h ^ (x & 1)) + 32 * (x >> 1);  // ^ (32 ks) gives chunk 2ks+h
    }
    // V reads (transposing): 16-lane group g4, lane i in the group reads row
    // 8h + rho (+ tile offsets) at 8-byte piece 4(i&3) of d block db.  With
    // the 4(row&3) swizzle the 32 lanes of a half-wave touch 16 distinct
    // chunks, i.e. all 64 banks once.
    {
      const int g4 = lane >> 4, i = lane & 15;
      const int hh = g4 >> 1, dgrp = g4 & 1, rho = i >> 2, b = (i & 3) >> 1, half = i & 1;
      v_rd = (8 * hh + rho) * 256 + 64 * rho + 32 * dgrp + 16 * b + 8 * half;  // ^ (64 db)
    }
  }

  // ---- tile staging (direct to LDS) --------------------------------------
  // Own tile i of this group (global key tile 2i + grp) lives in K stage
  // i & 1, V stage i & 1 and position stage i % 3.  The softmax phase of own
  // tile s issues one batch -- K and positions of own tile s+2, V of own tile
  // s+1 -- and waits, at its end, for the batch of the previous softmax
  // phase, which the GEMM phase right after it reads.  Every load is an
  // untracked DMA (dma_tile_to_lds), so these explicit waits are the only ones.
  __device__ __forceinline__ void load_k_tile(int j, int stage) {
    dma_tile_to_lds(krs, lds_k + stage * TILE_BYTES + 4096 * gwave, k_ld_off[0], k_ld_off[1],
                    k_ld_off[2], k_ld_off[3], j * BN * 256 + 4096 * gwave);
  }
  __device__ __forceinline__ void load_v_tile(int j, int stage) {
    dma_tile_to_lds(vrs, lds_v + stage * TILE_BYTES + 4096 * gwave, v_ld_off, v_ld_off, v_ld_off,
                    v_ld_off, j * BN * 256 + 4096 * gwave);
  }
  // All four waves of the group write the same 256 bytes (identical data),
  // which keeps every wave's count of outstanding loads the same.
  __device__ __forceinline__ void load_pos(int j, int stage) {
    dma_words_to_lds(prs, lds_pos + stage * BN * 4, lane * 4, j * BN * 4);
  }
  // Waits until at most n of this wave's DMA loads are outstanding.
  __device__ __forceinline__ static void wait_loads(int n) {
    if (n == 9) __builtin_amdgcn_s_waitcnt(0x0f79);       // vmcnt(9)
    else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0f70);              // vmcnt(0)
  }

  // The first two K tiles and position tiles of a block (own tiles 0 and 1),
  // into K stages 0, 1 and position stages 0, 1.
  __device__ __forceinline__ void load_block_head(int n_own_b, int j0_b) {
    if (n_own_b > 0) {
      load_k_tile(j0_b + grp, 0);
      load_pos(j0_b + grp, 0);
    }
    if (n_own_b > 1) {
      load_k_tile(j0_b + G + grp, 1);
      load_pos(j0_b + G + grp, 1);
    }
  }

  // ---- MFMA pieces --------------------------------------------------------
  // Each operand is read from LDS three MFMAs ahead of its use: with four
  // waves of the CU reading at once, an LDS read takes longer than one
  // 32-cycle MFMA, so a read issued just one MFMA ahead stalls the matrix
  // pipe.  The scheduling groups (0x100: LDS reads, 0x008: MFMAs) fix that
  // order; the compiler would otherwise interleave one read per MFMA.
  template <int MASK, int N>
  __device__ __forceinline__ static void sched() {
    __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
  }
  __device__ __forceinline__ f32x16 qk(int stage, int kb) const {
    const uint8_t* base = sm.k[grp][stage] + kb * 32 * 256;
    f32x16 s = {};
    bf16x8 av[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) av[ks] = *(const bf16x8*)(base + (k_rd ^ (32 * ks)));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks], q[ks], s, 0, 0, 0);
    sched<0x100, 3>();
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      sched<0x008, 1>();
      sched<0x100, 1>();
    }
    sched<0x008, 3>();
    return s;
  }
  __device__ __forceinline__ void pv(int stage, int kb, const bf16x8 (&p)[2]) {
    const uint8_t* base = sm.v[grp][stage] + kb * 32 * 256;
    bf16x8 av[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int off = (v_rd ^ (64 * db)) + t * 16 * 256;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off + 4 * 256));
        // whole-vector assembly: element-wise __bf16 inserts were mis-lowered
        const s16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        av[t][db] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[t][db], p[t], o[db], 0, 0, 0);
    sched<0x100, 6>();  // two transposing reads per operand
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      sched<0x008, 1>();
      sched<0x100, 2>();
    }
    sched<0x008, 3>();
  }

  // Masks keys of one 32-key half to -inf: those after the query (position
  // above qpe) and those past the block's end (tile index >= nvalid, whose
  // loaded positions read as zero).  Accumulator register r of half kb holds
  // tile key 32kb + 8h + 16(r/8) + r%8.
  __device__ __forceinline__ void mask(f32x16& s, const int32_t* pos, int kb, int qpe,
                                       int nvalid) const {
    i32x4 kp4[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
      kp4[x] = *(const i32x4*)&pos[32 * kb + 8 * h + 16 * (x >> 1) + 4 * (x & 1)];
    // key index 32kb + 8h + c_r < nvalid  <=>  8h < nvalid - 32kb - c_r
    const int h8 = 8 * h;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lim = nvalid - 32 * kb - (16 * (r >> 3) + (r & 7));
      const int kp = kp4[r >> 2][r & 3];
      const bool vis = kp <= qpe && (!DOCS || kp >= qlo) && h8 < lim;
      s[r] = vis ? s[r] : -INFINITY;
    }
  }

  __device__ __forceinline__ void exp_pack(const f32x16& s, float muse, bf16x8 (&p)[2]) {
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = fast_exp2(__builtin_fmaf(s[r], c2, -muse));
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) p[t][e] = (__bf16)x[8 * t + e];
    // four chains started from their first term: 12 adds, 3 to combine
    float a0 = x[0], a1 = x[1], a2 = x[2], a3 = x[3];
#pragma unroll
    for (int r = 4; r < 16; r += 4) {
      a0 += x[r];
      a1 += x[r + 1];
      a2 += x[r + 2];
      a3 += x[r + 3];
    }
    lsum += (a0 + a1) + (a2 + a3);
  }

  // Empty asm statements that make the phase's results exist at this point:
  // without them the compiler sinks pure arithmetic (exponentials, MFMAs)
  // into the next phase, next to its first use, and the phases blur.
  __device__ __forceinline__ void pin_softmax() {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) asm volatile("" : "+v"(pp[t][u]));
    asm volatile("" : "+v"(lsum), "+v"(m2), "+v"(alpha));
  }
  __device__ __forceinline__ void pin_gemm() {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(sc[kb]));
#pragma unroll
    for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(o[db]));
  }

  // Workgroup barrier that also stops the compiler from moving any
  // instruction across it, so each phase keeps its own work.
  __device__ __forceinline__ static void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- the two phases -----------------------------------------------------
  // Softmax of own tile s: classify the tile, mask, fold its row maximum into
  // the running maximum (rescaling O and l only when some row's maximum
  // rose), and turn the scores into bf16 probabilities.
  __device__ __forceinline__ void sm_phase(int s) {
    // The batch's DMA instructions are spread over the phase: a wave that
    // issues them back to back stalls on the CU's load path (64 B/clk).
    const bool has_k = s + 2 < n_own, has_v = s + 1 < n_own;
    if (has_k) load_k_tile(tile0() + G * (s + 2) + grp, s & 1);
    __builtin_amdgcn_sched_barrier(0);

    const int j = tile0() + G * s + grp;
    const int nvalid = min(BN, n_k - j * BN);
    const bool skip = j >= n_vis_w || (DOCS && j < lo_vis_w);
    const bool full = j < n_full_w && (!DOCS || j >= lo_full_w);
    if (!skip) {
      if (full) ++cnt_full; else ++cnt_masked;
    }
    if (skip) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[0][r] = sc[1][r] = -INFINITY;
    } else if (!full || nvalid < BN) {
      const int32_t* pos = sm.pos[grp][s % 3];
      mask(sc[0], pos, 0, qp, nvalid);
      mask(sc[1], pos, 1, qp, nvalid);
    }
    // four chains of three-input maxima over the 32 scores (v_max3: fewer
    // VALU instructions, which matters where the chip is power-limited)
    float mx4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& x = sc[c >> 1];
      const int o = 8 * (c & 1);
      float m = __builtin_fmaxf(__builtin_fmaxf(x[o], x[o + 1]), x[o + 2]);
      m = __builtin_fmaxf(__builtin_fmaxf(m, x[o + 3]), x[o + 4]);
      m = __builtin_fmaxf(__builtin_fmaxf(m, x[o + 5]), x[o + 6]);
      mx4[c] = __builtin_fmaxf(m, x[o + 7]);
    }
    const float mx = __builtin_fmaxf(__builtin_fmaxf(mx4[0], mx4[1]), __builtin_fmaxf(mx4[2], mx4[3]));
    const float mloc = half_swap_max(mx) * c2;
    // O is rescaled in the next GEMM phase, where the VALU is otherwise idle.
    resc = __ballot(mloc > m2) != 0;
    if (resc) {
      const float mnew = fmaxf(m2, mloc);
      alpha = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
    }
    const float muse = (m2 == -INFINITY) ? 0.f : m2;
    __builtin_amdgcn_sched_barrier(0);
    if (has_v) load_v_tile(tile0() + G * (s + 1) + grp, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    exp_pack(sc[0], muse, pp[0]);
    __builtin_amdgcn_sched_barrier(0);
    if (has_k) load_pos(tile0() + G * (s + 2) + grp, (s + 2) % 3);
    __builtin_amdgcn_sched_barrier(0);
    exp_pack(sc[1], muse, pp[1]);
    pin_softmax();
    wait_loads(has_k ? 9 : has_v ? 4 : 0);
  }

  // GEMM phase after the softmax of own tile s: the scores of own tile s+1
  // (S^T = K Q^T) and O += P(s) V(s).  s = -1 computes only the scores of
  // own tile 0; the last phase only PV.
  //
  // The wave in its GEMM phase runs at raised issue priority: when both waves
  // of a SIMD have an instruction ready, its MFMAs and their operand reads go
  // first, so the matrix pipe stays fed and the softmax wave's VALU work fills
  // the cycles in between.
  template <bool PV, bool QK>
  __device__ __forceinline__ void gemm_phase(int s) {
    __builtin_amdgcn_s_setprio(1);
    if (PV && !QK) prefetch_next_head();
    if (QK) {
      sc[0] = qk((s + 1) & 1, 0);
      sc[1] = qk((s + 1) & 1, 1);
    }
    if (PV) {
      if (resc) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
      }
      pv(s & 1, 0, pp[0]);
      pv(s & 1, 1, pp[1]);
    }
    pin_gemm();
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- one run: a query tile (128 rows of one head) against blocks --------
  int row = 0, n_kt = 0, n_kt_g = 0, qmax_wg = 0;
  size_t srow = 0;
  // First state row of this workgroup's slot when the key blocks are split
  // over several workgroups (each split writes its own partial state).
  size_t slot_rows = 0;
  // Write out/lse rather than the state even though FINAL is false (a tile
  // of the split launch that is folded whole).
  bool final_rt = false;
  float m_nat0 = -INFINITY, m2_0 = -INFINITY;
  bool count = false;

  // Query positions of the tile: the wave's first and last position and the
  // workgroup's last (positions increase within the array).
  __device__ __forceinline__ void positions(int qt, int head) {
    const int row0_wg = qt * ROWS;
    const int row0 = row0_wg + gwave * WAVE_ROWS;
    wave_valid = row0 < n_q;
    row = row0 + col;
    if (!wave_valid) {
      qmin_w = qmax_w = kPosRowNone;
    } else if (!causal) {
      qmin_w = qmax_w = kPosRowAll;
    } else {
      qmin_w = __builtin_amdgcn_readfirstlane(a.q_pos[row0]);
      qmax_w = __builtin_amdgcn_readfirstlane(a.q_pos[min(row0 + WAVE_ROWS, n_q) - 1]);
    }
    qmax_wg = causal ? a.q_pos[min(row0_wg + ROWS, n_q) - 1] : kPosRowAll;
    qp = row < n_q ? (causal ? a.q_pos[row] : kPosRowAll) : kPosRowNone;
    if (DOCS) {
      // Lower bounds never decrease along the rows (documents follow the
      // positions), so first and last rows give the extremes.
      qlo_min_wg = a.q_lo[row0_wg];
      if (wave_valid) {
        qlo_min_w = __builtin_amdgcn_readfirstlane(a.q_lo[row0]);
        qlo_max_w = __builtin_amdgcn_readfirstlane(a.q_lo[min(row0 + WAVE_ROWS, n_q) - 1]);
      }
      qlo = row < n_q ? a.q_lo[row] : kPosLoNone;
    }
    count = a.work != nullptr && head == 0 && wave_valid;
    srow = slot_rows + (size_t)head * n_q + row;
  }

  // Tile classes of one key block from one pass over its positions.
  // Positions increase, so the key tiles the workgroup sees form a prefix of
  // the block (n_iter tiles), and so do the tiles this wave sees completely
  // (n_full_w) and at all (n_vis_w).
  // With lower bounds (document starts) the tiles seen also start late:
  // those whose last key lies before a bound form a prefix too, so each set
  // is a range [lo, end) of tiles.  The workgroup visits [j0, n_iter_end),
  // j0 its first visible tile rounded down to even; n_iter counts from j0.
  struct Classes {
    int n_iter, n_full_w, n_vis_w, j0, lo_full_w, lo_vis_w;
  };
  __device__ __forceinline__ Classes classes_of(const int32_t* k_pos) const {
    const int nkt = (n_k + BN - 1) / BN;
    Classes c{nkt, 0, 0, 0, 0, 0};
    if (causal) {
      int ci = 0, cf = 0, cv = 0, li = 0, lf = 0, lv = 0;
      for (int j = lane; j < nkt; j += 64) {
        const int kf = k_pos[j * BN];
        const int kl = k_pos[min(j * BN + BN, n_k) - 1];
        ci += kf <= qmax_wg ? 1 : 0;
        cf += kl <= qmin_w ? 1 : 0;
        cv += kf <= qmax_w ? 1 : 0;
        if (DOCS) {
          li += kl < qlo_min_wg ? 1 : 0;
          lf += kf < qlo_max_w ? 1 : 0;
          lv += kl < qlo_min_w ? 1 : 0;
        }
      }
      const int n_end = __builtin_amdgcn_readfirstlane(wave_sum_i(ci));
      c.n_full_w = wave_valid ? __builtin_amdgcn_readfirstlane(wave_sum_i(cf)) : 0;
      c.n_vis_w = wave_valid ? __builtin_amdgcn_readfirstlane(wave_sum_i(cv)) : 0;
      if (DOCS) {
        c.j0 = __builtin_amdgcn_readfirstlane(wave_sum_i(li)) & ~1;
        c.lo_full_w = __builtin_amdgcn_readfirstlane(wave_sum_i(lf));
        c.lo_vis_w = __builtin_amdgcn_readfirstlane(wave_sum_i(lv));
      }
      c.n_iter = DOCS ? max(0, n_end - c.j0) : n_end;
    } else {
      c.n_full_w = c.n_vis_w = wave_valid ? nkt : 0;
    }
    return c;
  }
  // This group's own tiles among n_iter visited key tiles.
  __device__ __forceinline__ int own_tiles(int n_it) const {
    return (n_it - grp + G - 1) / G;
  }
  __device__ __forceinline__ void use_classes(const Classes& c) {
    n_kt = (n_k + BN - 1) / BN;
    n_iter = c.n_iter;
    n_full_w = c.n_full_w;
    n_vis_w = c.n_vis_w;
    j0 = c.j0;
    lo_full_w = c.lo_full_w;
    lo_vis_w = c.lo_vis_w;
    // tiles of this group among all key tiles, and among the visited ones
    n_kt_g = (n_kt - grp + G - 1) / G;
    n_own = own_tiles(n_iter);
  }
  __device__ __forceinline__ void classify(const int32_t* k_pos) { use_classes(classes_of(k_pos)); }

  // Next block of an all-gather run: its buffers and tile classes, and
  // whether this group already issued the loads of its first tiles.
  const void* nxt_k = nullptr;
  const int32_t* nxt_pos = nullptr;
  int nxt_own = 0, nxt_kvh = 0, nxt_j0 = 0;
  bool head_issued = false;

  // Issued by the last GEMM phase of a block (PV only: the K stages are idle
  // and the position stages were last read by the softmax phase before it):
  // K and positions of the next block's first two own tiles.
  __device__ __forceinline__ void prefetch_next_head() {
    if (nxt_k == nullptr || nxt_own == 0) return;
    krs = buffer_rsrc((const uint16_t*)nxt_k + ((size_t)nxt_kvh * n_k) * D, n_k * D * 2);
    prs = buffer_rsrc(nxt_pos, n_k * 4);
    load_block_head(nxt_own, DOCS ? nxt_j0 : 0);
    head_issued = true;
  }

  // Q into registers and the incoming state (READ) or the empty one.
  __device__ __forceinline__ void load_state(int head) {
    {
      const uint16_t* qb = (const uint16_t*)a.q + ((size_t)head * n_q) * D;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        q[ks] = row < n_q ? *(const bf16x8*)(qb + (size_t)row * D + ks * 16 + h * 8) : bf16x8{};
    }
    m_nat0 = -INFINITY;
    m2 = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    // Group 0 carries the incoming state.  Group 1 starts with empty sums but
    // the same reference max, so its first tiles do not trigger rescales
    // (any reference at or above the scores seen gives the same softmax).
    if (READ && row < n_q) {
      m_nat0 = a.m_in[srow];
      m2 = m_nat0 * kLog2e;
    }
    if (READ && grp == 0 && row < n_q) {
      lsum = h == 0 ? a.l_in[srow] : 0.f;
      const float* orow = a.o_in + srow * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x = *(const f32x4*)(orow + db * 32 + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][4 * g + e] = x[e];
        }
    }
    m2_0 = m2;
    c2 = a.c2;
    resc = false;
  }

  // Folds one key/value block (already classified) into the running state.
  // Ping-pong schedule.  Each group alternates softmax phases (VALU) and
  // GEMM phases (MFMA) on its own tiles, one workgroup barrier after each
  // phase.  Group 1 starts one phase later, so on every SIMD one wave feeds
  // the matrix pipe while the other runs the softmax, and each barrier
  // swaps their roles.  Group g passes g + 1 + 2 n_own barriers after the
  // prologue and pads to the larger count of the two.  Every wave of the
  // workgroup takes the same branches (n_iter is workgroup-uniform).
  __device__ __forceinline__ void fold_block(const void* k, const void* v, const int32_t* k_pos,
                                             int kvh) {
    cnt_full = cnt_masked = 0;
    if (n_iter > 0) {
      kbase = (const uint16_t*)k + ((size_t)kvh * n_k) * D;
      vbase = (const uint16_t*)v + ((size_t)kvh * n_k) * D;
      krs = buffer_rsrc(kbase, n_k * D * 2);
      vrs = buffer_rsrc(vbase, n_k * D * 2);
      prs = buffer_rsrc(k_pos, n_k * 4);
      if (!head_issued) load_block_head(n_own, tile0());
      head_issued = false;
      // V of own tile 0 is first read two phases on; the softmax phase of
      // own tile 0 waits for it.  Everything older must land now.
      if (n_own > 0) {
        load_v_tile(tile0() + grp, 0);
        wait_loads(4);
      } else {
        wait_loads(0);
      }
      phase_barrier();
      if (G == 2 && grp == 1) phase_barrier();
      if (n_own > 0) gemm_phase<false, true>(-1);
      phase_barrier();
      for (int s = 0; s + 1 < n_own; ++s) {
        sm_phase(s);
        phase_barrier();
        gemm_phase<true, true>(s);
        phase_barrier();
      }
      if (n_own > 0) {
        sm_phase(n_own - 1);
        phase_barrier();
        gemm_phase<true, false>(n_own - 1);
        phase_barrier();
      }
      if (G == 2) {
        const int n0 = (n_iter + 1) / 2, n1 = n_iter / 2;
        const int n_bar = max(2 * n0 + 1, 2 * n1 + 2);
        for (int b = grp + 1 + 2 * n_own; b < n_bar; ++b) phase_barrier();
      }
    }
    if (count && lane == 0) {
      atomicAdd(a.work + 0, (unsigned long long)cnt_full);
      atomicAdd(a.work + 1, (unsigned long long)cnt_masked);
      atomicAdd(a.work + 2, (unsigned long long)(n_kt_g - cnt_full - cnt_masked));
    }
  }

  // Folds group 1's partial state into group 0's through LDS and writes the
  // result: normalised out/lse (FINAL) or the running state.
  // Two groups: group 1's partial state folds into group 0's through LDS.
  __device__ __forceinline__ void merge_groups() {
    __syncthreads();  // every wave is done with the K/V stages
    float* mo = (float*)&sm.k[0][0][0];            // [wave][reg][lane] O^T values
    float* ml = mo + 4 * 64 * 64;                  // [wave][lane] m2, then lsum
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mo[(gwave * 64 + db * 16 + r) * 64 + lane] = o[db][r];
      ml[gwave * 64 + lane] = m2;
      ml[4 * 64 + gwave * 64 + lane] = lsum;
    }
    __syncthreads();
    if (grp == 0) {
      const float m2b = ml[gwave * 64 + lane];
      const float lb = ml[4 * 64 + gwave * 64 + lane];
      const float mn = fmaxf(m2, m2b);
      const float fa = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mn);
      const float fb = (m2b == -INFINITY) ? 0.f : fast_exp2(m2b - mn);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o[db][r] = o[db][r] * fa + mo[(gwave * 64 + db * 16 + r) * 64 + lane] * fb;
      lsum = lsum * fa + lb * fb;
      m2 = mn;
    }
  }

  __device__ __forceinline__ void finish() {
    if constexpr (G == 2) merge_groups();
    if (grp == 1) return;

    const float ltot = half_swap_sum(lsum);
    if (row >= n_q) return;
    const float m_nat = (m2 == m2_0) ? m_nat0 : m2 * kLn2;
    if (FINAL || final_rt) {
      const bool ok = ltot > 0.f;
      const float inv = ok ? 1.f / ltot : 0.f;
      float* orow = a.out + srow * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
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
      for (int db = 0; db < 4; ++db)
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

  // One ring step: the query tile against the block in a.k / a.v.
  __device__ void run(int qt, int head) {
    positions(qt, head);
    classify(a.k_pos);
    if (READ && !FINAL && n_iter == 0) {
      // nothing visible: the state stays as it is
      if (count && lane == 0) atomicAdd(a.work + 2, (unsigned long long)n_kt_g);
      return;
    }
    load_state(head);
    fold_block(a.k, a.v, a.k_pos, head / (a.h_q / a.h_kv));
    finish();
  }

  // Consecutive ring blocks in one launch (up to kChunkBlocks, one group per
  // workgroup), the running state in registers between them.  Between two
  // blocks it goes through the same rounding as a store and reload between
  // two step launches (the max in natural log, the row sum gathered in one
  // half-wave), so the result is bit for bit that of one launch per block;
  // a tile that sees none of the blocks leaves the state untouched.
  __device__ void run_chunk(const MultiArgs& ma, int qt, int head) {
    static_assert(G == 1, "one group per workgroup");
    positions(qt, head);
    Classes cls[kChunkBlocks];
    bool any = false;
#pragma unroll
    for (int b = 0; b < kChunkBlocks; ++b) {
      if (b < ma.n_blocks) {
        cls[b] = classes_of(ma.k_pos[b]);
        any = any || cls[b].n_iter > 0;
      }
    }
    if (READ && !FINAL && !any) {
      if (count && lane == 0) {
        const int n_kt_all = (n_k + BN - 1) / BN;
        atomicAdd(a.work + 2, (unsigned long long)(ma.n_blocks * n_kt_all));
      }
      return;
    }
    load_state(head);
    const int kvh = head / (a.h_q / a.h_kv);
    head_issued = false;
    nxt_kvh = kvh;  // the prefetch of the next block's first tiles reads this head
#pragma unroll
    for (int b = 0; b < kChunkBlocks; ++b) {
      if (b < ma.n_blocks) {
        use_classes(cls[b]);
        if (b + 1 < ma.n_blocks) {
          nxt_k = ma.k[b + 1];
          nxt_pos = ma.k_pos[b + 1];
          nxt_own = own_tiles(cls[b + 1].n_iter);
        } else {
          nxt_k = nullptr;
          nxt_pos = nullptr;
          nxt_own = 0;
        }
        fold_block(ma.k[b], ma.v[b], ma.k_pos[b], kvh);
        if (b + 1 < ma.n_blocks) {
          // the store and reload between two step launches, in registers
          const float ltot = half_swap_sum(lsum);
          const float m_nat = (m2 == m2_0) ? m_nat0 : m2 * kLn2;
          m_nat0 = m_nat;
          m2 = m_nat * kLog2e;
          m2_0 = m2;
          lsum = h == 0 ? ltot : 0.f;
          resc = false;
        }
      }
    }
    nxt_k = nullptr;
    finish();
  }

  // All blocks resident: the query tile against every block in turn, the
  // running state staying in registers between them.  Under a document mask
  // only the blocks b with b mod n_split = split are folded.
  __device__ void run_all(const MultiArgs& ma, int qt, int head, int split = 0, int n_split = 1) {
    positions(qt, head);
    load_state(head);
    const int kvh = head / (a.h_q / a.h_kv);
    head_issued = false;
    nxt_kvh = kvh;
    if constexpr (DOCS) {
      if (!run_blocks_screened(ma, kvh, split, n_split) && !FINAL && !final_rt) {
        // No block of this split can hold a visible key: the partial state
        // is empty, which its max alone records (the merge reads nothing else).
        if (grp == 0 && h == 0 && row < n_q) a.m_out[srow] = -INFINITY;
        return;
      }
    } else {
      Classes cur = ma.n_blocks > 0 ? classes_of(ma.k_pos[0]) : Classes{0, 0, 0, 0, 0, 0};
      for (int b = 0; b < ma.n_blocks; ++b) {
        use_classes(cur);
        // the next block's classes (their loads overlap this block) and what
        // its first tiles need
        if (b + 1 < ma.n_blocks) {
          cur = classes_of(ma.k_pos[b + 1]);
          nxt_k = ma.k[b + 1];
          nxt_pos = ma.k_pos[b + 1];
          nxt_own = own_tiles(cur.n_iter);
        } else {
          nxt_k = nullptr;
          nxt_pos = nullptr;
          nxt_own = 0;
        }
        fold_block(ma.k[b], ma.v[b], ma.k_pos[b], kvh);
      }
    }
    nxt_k = nullptr;
    finish();
  }

  // Under a document mask most blocks hold no key a workgroup sees.  Lane b
  // checks block b's first key against the workgroup's last query and its
  // last key against the smallest document start; one ballot, the same in
  // every wave, then replaces a classification pass per hidden block.
  __device__ __forceinline__ bool run_blocks_screened(const MultiArgs& ma, int kvh, int split,
                                                      int n_split) {
    bool maybe = false;
    if (lane < ma.n_blocks && n_k > 0 && lane % n_split == split) {
      const int32_t* kp = ma.k_pos[lane];
      maybe = kp[0] <= qmax_wg && kp[n_k - 1] >= qlo_min_wg;
    }
    uint64_t todo = __ballot(maybe);
    const bool any = todo != 0;
    int b = todo ? __builtin_ctzll(todo) : -1;
    Classes cur = b >= 0 ? classes_of(ma.k_pos[b]) : Classes{0, 0, 0, 0, 0, 0};
    while (b >= 0) {
      use_classes(cur);
      todo &= todo - 1;
      const int nb = todo ? __builtin_ctzll(todo) : -1;
      if (nb >= 0) {
        cur = classes_of(ma.k_pos[nb]);
        nxt_k = ma.k[nb];
        nxt_pos = ma.k_pos[nb];
        nxt_own = own_tiles(cur.n_iter);
        nxt_j0 = cur.j0;
      } else {
        nxt_k = nullptr;
        nxt_pos = nullptr;
        nxt_own = 0;
      }
      fold_block(ma.k[b], ma.v[b], ma.k_pos[b], kvh);
      b = nb;
    }
    return any;
  }
};

template <int G, bool READ, bool FINAL>
__global__ __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(2, 2)))
void step_kernel_fast(const StepArgs a) {
  __shared__ Smem<G> sm;
  const int tid = threadIdx.x;
  const int u = blockIdx.x + a.unit0;
  const int head = a.head_of[u % a.h_q];
  const int p = u / a.h_q;
  const int t_hi = a.n_qt - 1 - p, t_lo = p;
  Step<G, READ, FINAL> s(a, sm, tid);
  s.run(t_hi, head);
  if (t_lo < t_hi) {
    __syncthreads();
    s.run(t_lo, head);
  }
}

// Up to kChunkBlocks consecutive ring blocks per launch (one group per
// workgroup): the units as in step_kernel_fast.
template <bool READ, bool FINAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void chunk_kernel_fast(const MultiArgs ma) {
  __shared__ Smem<1> sm;
  const int tid = threadIdx.x;
  const int u = blockIdx.x + ma.s.unit0;
  const int head = ma.s.head_of[u % ma.s.h_q];
  const int p = u / ma.s.h_q;
  const int t_hi = ma.s.n_qt - 1 - p, t_lo = p;
  Step<1, READ, FINAL> s(ma.s, sm, tid);
  s.run_chunk(ma, t_hi, head);
  if (t_lo < t_hi) {
    __syncthreads();
    s.run_chunk(ma, t_lo, head);
  }
}

// All-gather form: every key/value block resident, one launch.  DOCS: each
// query's keys are also bounded below by its document start (a.q_lo).
template <int G, bool DOCS>
__global__ __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(2, 2)))
void allgather_kernel_fast(const MultiArgs ma) {
  __shared__ Smem<G> sm;
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int head = ma.s.head_of[u % ma.s.h_q];
  const int p = u / ma.s.h_q;
  const int t_hi = ma.s.n_qt - 1 - p, t_lo = p;
  Step<G, false, true, DOCS> s(ma.s, sm, tid);
  s.run_all(ma, t_hi, head);
  if (t_lo < t_hi) {
    __syncthreads();
    s.run_all(ma, t_lo, head);
  }
}

// Two chains of the all-gather form: one-group workgroups fold the blocks
// in `ma` (one parity of the block list) into partial state `chain` of the
// state arrays (chain x h_q x n_q rows in), which merge_splits_kernel<true>
// combines after both chains; the two launches run side by side, two
// workgroups to a compute unit.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void allgather_chain_kernel_fast(const MultiArgs ma, int chain) {
  __shared__ Smem<1> sm;
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int head = ma.s.head_of[u % ma.s.h_q];
  const int p = u / ma.s.h_q;
  const int t_hi = ma.s.n_qt - 1 - p, t_lo = p;
  Step<1, false, false> s(ma.s, sm, tid);
  s.slot_rows = (size_t)chain * ma.s.h_q * ma.s.n_q;
  s.run_all(ma, t_hi, head);
  if (t_lo < t_hi) {
    __syncthreads();
    s.run_all(ma, t_lo, head);
  }
}

// The same under a document mask with the key blocks split over n_split
// workgroups per query tile pair.  A tile whose rows see a long span of
// positions (late rows of a long document) is split: split s folds the blocks
// b with b mod n_split = s into a partial state (m, l, O) in slot s of the
// state arrays, and merge_splits_kernel combines them.  That walk then no
// longer sets the length of the whole launch, and consecutive chunks of one
// document (held by different blocks) go to different splits.  Other tiles
// are folded whole by split 0, which writes out and lse itself.
//
// Every global position lies in exactly one block, so a tile's walk over all
// blocks is about (last row's position - first row's document start) / 64
// key tiles; a tile is split when that span exceeds kSplitSpan positions.
__device__ __forceinline__ bool split_tile(const int32_t* q_pos, const int32_t* q_lo, int n_q,
                                           int t) {
  const int last = min((t + 1) * ROWS, n_q) - 1;
  return q_pos[last] - q_lo[t * ROWS] > kSplitSpan;
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void allgather_split_kernel_fast(const MultiArgs ma, int n_split) {
  __shared__ Smem<2> sm;
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int sp = blockIdx.y;
  const int head = ma.s.head_of[u % ma.s.h_q];
  const int p = u / ma.s.h_q;
  const int t_hi = ma.s.n_qt - 1 - p, t_lo = p;
  Step<2, false, false, true> s(ma.s, sm, tid);
  for (int k = 0; k < 2; ++k) {
    const int t = k == 0 ? t_hi : t_lo;
    if (k == 1) {
      if (t_lo >= t_hi) break;
      __syncthreads();
    }
    const bool split = split_tile(ma.s.q_pos, ma.s.q_lo, ma.s.n_q, t);
    if (!split && sp != 0) continue;
    s.final_rt = !split;
    s.slot_rows = split ? (size_t)sp * ma.s.h_q * ma.s.n_q : 0;
    s.run_all(ma, t, head, split ? sp : 0, split ? n_split : 1);
  }
}

// Combines the n_split partial states of each row of a split tile (slot s at
// m + s rows, l + s rows, o + s rows * D) with the online-softmax rescale and
// writes the normalised out and lse: M = max_s m_s, L = sum_s l_s e^(m_s - M),
// out = sum_s O_s e^(m_s - M) / L, lse = M + ln L.  A slot whose max is -inf
// saw no key and is not read further.  Rows of tiles that were not split
// already hold their result (ALL: every row is merged, q_pos and q_lo unused).
// One wave per row, two columns a lane.
constexpr int MERGE_ROWS = 4;
template <bool ALL>
__global__ __launch_bounds__(64 * MERGE_ROWS)
void merge_splits_kernel(const float* __restrict__ m, const float* __restrict__ l,
                         const float* __restrict__ o, const int32_t* __restrict__ q_pos,
                         const int32_t* __restrict__ q_lo, int n_q, int n_split, long long rows,
                         float* __restrict__ out, float* __restrict__ lse) {
  const long long r = (long long)blockIdx.x * MERGE_ROWS + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  if (!ALL && !split_tile(q_pos, q_lo, n_q, (int)(r % n_q) / ROWS)) return;
  const float ms = lane < n_split ? m[lane * rows + r] : -INFINITY;
  float mx = ms;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  uint64_t seen = __ballot(ms != -INFINITY);
  float lt = 0.f, o0 = 0.f, o1 = 0.f;
  while (seen) {
    const int s = __builtin_ctzll(seen);
    seen &= seen - 1;
    const float w = expf(__shfl(ms, s) - mx);
    const long long sr = s * rows + r;
    lt += w * l[sr];
    const float2 x = *(const float2*)(o + sr * D + 2 * lane);
    o0 += w * x.x;
    o1 += w * x.y;
  }
  const bool ok = lt > 0.f;
  const float inv = ok ? 1.f / lt : 0.f;
  *(float2*)(out + r * D + 2 * lane) = float2{o0 * inv, o1 * inv};
  if (lane == 0) lse[r] = ok ? mx + logf(lt) : -INFINITY;
}

}  // namespace fast

hipError_t launch_allgather_split_fast(const MultiArgs& ma, int n_split, hipStream_t stream) {
  dim3 grid((unsigned)(ma.s.n_pairs * ma.s.h_q), (unsigned)n_split), block(fast::threads<2>());
  hipLaunchKernelGGL(fast::allgather_split_kernel_fast, grid, block, 0, stream, ma, n_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)ma.s.h_q * ma.s.n_q;
  dim3 mgrid((unsigned)((rows + fast::MERGE_ROWS - 1) / fast::MERGE_ROWS)),
      mblock(64 * fast::MERGE_ROWS);
  hipLaunchKernelGGL(fast::merge_splits_kernel<false>, mgrid, mblock, 0, stream, ma.s.m_out,
                     ma.s.l_out, ma.s.o_out, ma.s.q_pos, ma.s.q_lo, ma.s.n_q, n_split, rows,
                     ma.s.out, ma.s.lse);
  return hipGetLastError();
}

hipError_t launch_merge_states(const float* m, const float* l, const float* o, long long rows,
                               int n_states, float* out, float* lse, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  dim3 mgrid((unsigned)((rows + fast::MERGE_ROWS - 1) / fast::MERGE_ROWS)),
      mblock(64 * fast::MERGE_ROWS);
  hipLaunchKernelGGL(fast::merge_splits_kernel<true>, mgrid, mblock, 0, stream, m, l, o, nullptr,
                     nullptr, 0, n_states, rows, out, lse);
  return hipGetLastError();
}

// Groups per workgroup for a launch of `units` workgroup-sized work units
// (query tile pairs x heads): one group when there are at least two units per
// compute unit, so that two one-group workgroups share each compute unit;
// otherwise the two-group ping-pong keeps both waves of a SIMD busy.
static int groups_for(long long units) {
  // compute units of the current device, looked up once per device
  static std::atomic<int> cus_of[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cus_of[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    int n = 0;
    cus = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                  n > 0
              ? n
              : 256;
    cus_of[dev].store(cus, std::memory_order_relaxed);
  }
  return units >= 2LL * cus ? 1 : 2;
}

int fast_groups_for(long long units) { return groups_for(units); }

// Two chains of one-group launches (even blocks into one state, odd blocks
// into another, on two streams) fill the chip where one chain of one-group
// workgroups would leave a compute unit with a single one: at least one
// work unit per compute unit, fewer than two.
bool fast_two_chains(long long units) {
  return groups_for(units) == 2 && groups_for(2 * units) == 1;
}

hipError_t launch_allgather_fast(const MultiArgs& ma, hipStream_t stream) {
  const int g = ma.s.q_lo != nullptr ? 2 : groups_for((long long)ma.s.n_pairs * ma.s.h_q);
  dim3 grid((unsigned)(ma.s.n_pairs * ma.s.h_q)), block(256 * g);
  if (ma.s.q_lo != nullptr)
    hipLaunchKernelGGL((fast::allgather_kernel_fast<2, true>), grid, block, 0, stream, ma);
  else if (g == 1)
    hipLaunchKernelGGL((fast::allgather_kernel_fast<1, false>), grid, block, 0, stream, ma);
  else
    hipLaunchKernelGGL((fast::allgather_kernel_fast<2, false>), grid, block, 0, stream, ma);
  return hipGetLastError();
}

hipError_t launch_allgather_chain_fast(const MultiArgs& ma, int chain, hipStream_t stream) {
  dim3 grid((unsigned)(ma.s.n_pairs * ma.s.h_q)), block(256);
  hipLaunchKernelGGL(fast::allgather_chain_kernel_fast, grid, block, 0, stream, ma, chain);
  return hipGetLastError();
}

hipError_t launch_chunk_fast(const MultiArgs& ma, bool read, bool final_, hipStream_t stream) {
  const StepArgs& a = ma.s;
  dim3 grid((unsigned)(a.n_units ? a.n_units : a.n_pairs * a.h_q)), block(256);
  if (read && final_)
    hipLaunchKernelGGL((fast::chunk_kernel_fast<true, true>), grid, block, 0, stream, ma);
  else if (read)
    hipLaunchKernelGGL((fast::chunk_kernel_fast<true, false>), grid, block, 0, stream, ma);
  else if (final_)
    hipLaunchKernelGGL((fast::chunk_kernel_fast<false, true>), grid, block, 0, stream, ma);
  else
    hipLaunchKernelGGL((fast::chunk_kernel_fast<false, false>), grid, block, 0, stream, ma);
  return hipGetLastError();
}

template <int G>
static void launch_step_g(const StepArgs& a, bool read, bool final_, hipStream_t stream,
                          hipEvent_t start, hipEvent_t stop) {
  dim3 grid((unsigned)(a.n_units ? a.n_units : a.n_pairs * a.h_q)), block(256 * G);
  auto go = [&](auto kernel) {
    if (start || stop)
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, a);
    else
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, a);
  };
  if (read && final_)
    go(fast::step_kernel_fast<G, true, true>);
  else if (read)
    go(fast::step_kernel_fast<G, true, false>);
  else if (final_)
    go(fast::step_kernel_fast<G, false, true>);
  else
    go(fast::step_kernel_fast<G, false, false>);
}

hipError_t launch_step_fast(const StepArgs& a, bool read, bool final_, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop) {
  if ((a.groups ? a.groups : groups_for((long long)a.n_pairs * a.h_q)) == 1)
    launch_step_g<1>(a, read, final_, stream, start, stop);
  else
    launch_step_g<2>(a, read, final_, stream, start, stop);
  return hipGetLastError();
}

}  // namespace ra
