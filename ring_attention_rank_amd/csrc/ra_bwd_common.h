// Shared pieces of the backward kernels (bfloat16, d_k = 128, gfx950): MFMA
// operand layouts, LDS swizzles and tile staging.  Included by the dq and
// the dk/dv translation units, which are compiled with different register
// forms for the MFMA accumulators.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
constexpr int ROWS = 128;      // rows a workgroup owns (4 wave pairs x 32)
constexpr int TILE = 64;       // rows of a staged tile
constexpr int TILE_BYTES = TILE * D * 2;  // 16 KiB
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }

// XCD-aware split of a one-dimensional grid of n_x * n_y workgroups into
// (x, y).  Workgroup L runs on XCD L % 8 (8 XCDs, each with its own L2); when
// n_y is a multiple of 8, XCD c gets the contiguous y range
// [c n_y / 8, (c + 1) n_y / 8), so the workgroups that share data through y
// (a key/value head, a head-group split) meet in one L2.
__device__ __forceinline__ void xcd_split(int L, int n_y, int& x, int& y) {
  if ((n_y & 7) == 0) {
    const int per = n_y >> 3, rest = L >> 3;
    y = (L & 7) * per + rest % per;
    x = rest / per;
  } else {
    y = L % n_y;
    x = L / n_y;
  }
}

// Buffer resource over `bytes` bytes at `base`: loads past the end return
// zero without a branch, so every wave issues the same loads and the
// compiler can count them (it waits for the oldest ones only).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Register value r of half kb of an S^T or S accumulator belongs to tile row
// 32 kb + 8 h + 16 (r / 8) + r % 8.
__device__ __forceinline__ int acc_row(int kb, int h, int r) {
  return 32 * kb + 8 * h + 16 * (r >> 3) + (r & 7);
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

// ---- one-copy tiles (LDS DMA) ------------------------------------------
// A tile staged once and read both ways: 16-byte chunk c of row r sits at
// physical chunk c ^ uswz(r).  uswz is a bijection on r & 15 (row reads of 16
// rows with the same chunk hit 16 distinct chunks) whose bits 2-3 take all
// four values over any four rows 4k .. 4k + 3 (the 4 rows x 4 chunks a
// half-wave of transposing reads touches hit 16 distinct chunks): both read
// patterns are free of bank conflicts.
__device__ __forceinline__ int uswz(int r) { return 4 * (r & 3) | ((r >> 2) & 3); }

// Per-lane read bases into a one-copy tile.  Row reads of half kb take row
// sigma(col) + 32 kb, logical chunk 2 ks + h (the MFMA A operand of 32 rows
// x 16 columns, rows permuted by sigma as in the forward kernel); the
// transposing reads give the 32 x 16 operand of d block db and row group t
// of half kb in two ds_read_b64_tr_b16 (rows 8 hh + rho and 4 rows on).
struct Lanes1 {
  int rd_row, rd_lo, rd_hi, h, col;
  __device__ Lanes1(int lane) {
    h = lane >> 5;
    col = lane & 31;
    const int r = sigma(col), g = uswz(r);
    rd_row = r * 256 + 16 * (h ^ (g & 1)) + 32 * (g >> 1);  // ^ (32 ks)
    const int g4 = lane >> 4, i = lane & 15;
    const int hh = g4 >> 1, dgrp = g4 & 1, rho = i >> 2, b = (i & 3) >> 1, half = i & 1;
    const int c = 2 * dgrp + b;
    rd_lo = (8 * hh + rho) * 256 + 64 * rho + 16 * (c ^ (2 * hh)) + 8 * half;          // ^ (64 db)
    rd_hi = (8 * hh + rho + 4) * 256 + 64 * rho + 16 * (c ^ (2 * hh + 1)) + 8 * half;  // ^ (64 db)
  }
};

__device__ __forceinline__ bf16x8 row_operand1(const uint8_t* tile, const Lanes1& L, int kb,
                                               int ks) {
  return *(const bf16x8*)(tile + kb * 32 * 256 + (L.rd_row ^ (32 * ks)));
}
__device__ __forceinline__ bf16x8 tr_operand1(const uint8_t* tile, const Lanes1& L, int kb, int t,
                                              int db) {
  const uint8_t* base = tile + kb * 32 * 256 + t * 16 * 256;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + (L.rd_lo ^ (64 * db))));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + (L.rd_hi ^ (64 * db))));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Buffer resource as four wave-uniform words, for the inline LDS DMA below
// (reads at or past `bytes` return zeros).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xffff),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// Eight rows (2 KiB) from HBM straight into LDS: load i of lane L reads
// global byte soff + 1024 i + v_i and lands at LDS byte lds + 1024 i + 16 L.
// Inline asm, so the compiler does not track these loads (it would wait for
// them before the next LDS read of the other stage); the caller waits with
// vmcnt before the barrier that publishes the stage.  M0 carries the LDS
// address, and the nop is the wait state between writing M0 and its use.
__device__ __forceinline__ void dma_rows8(const i32x4& rs, uint32_t lds, int v0, int v1,
                                          int soff) {
  const int m0v = __builtin_amdgcn_readfirstlane((int)lds);
  const int so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds"
      :
      : "s"(m0v), "v"(v0), "v"(v1), "s"(rs), "s"(so)
      : "m0");
}

// One 4-byte word per lane (256 bytes) from HBM straight into LDS: lane L's
// word lands at lds + 4 L (same conventions as dma_rows8).
__device__ __forceinline__ void dma_words64(const i32x4& rs, uint32_t lds, int voff, int soff) {
  const int m0v = __builtin_amdgcn_readfirstlane((int)lds);
  const int so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rs), "s"(so)
               : "m0");
}

// Scheduling fence: the tile loops below are written in the order they
// should issue (each MFMA with the LDS reads four MFMAs ahead and a slice of
// the other half's VALU work) and the compiler keeps that order.
#define RA_FENCE() __builtin_amdgcn_sched_barrier(0)

}  // namespace bwd
}  // namespace ra
