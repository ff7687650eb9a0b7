// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ra.h"

namespace ra {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kWavesPerGroup = 4;  // one wave per SIMD of a CU
constexpr int kRowsPerWave = 32;   // query rows a wave owns (one 32-row MFMA block)
constexpr int kRowsPerGroup = kWavesPerGroup * kRowsPerWave;  // 128
constexpr int kKeysPerTile = 64;   // keys per LDS tile
constexpr int kMaxHeads = 256;
constexpr int kMaxBlocks = 64;     // key/value blocks of one all-gather launch
// Document-masked all-gather: a query tile whose rows span more than this
// many positions from its first row's document start to its last row is
// split over several workgroups (its walk over the blocks is long).
constexpr int kSplitSpan = 8192;

// The ring forward behind ra_forward / ra_forward_timed (arguments as
// there); fixed: null, or five caller-made events (no timing, no system
// fence) used in place of per-call ones; with them the workspace needs only
// the two-slot layout (the schedule then never chunks).
ra_status forward_ring(const ra_problem* p, int32_t n_cp, const void* q, const int32_t* q_pos,
                       const void* const* k_blocks, const void* const* v_blocks,
                       const int32_t* const* k_pos_blocks, void* workspace, size_t ws_bytes,
                       float* out, float* lse, int64_t* work, int64_t* staged_bytes,
                       void* main_stream, void* side_stream, void* const* launch_events,
                       void* const* staged_events, const hipEvent_t* fixed);
// Bytes of the no-alloc form's workspace (one state, two staging slots); 0
// for an invalid problem.
size_t forward_noalloc_bytes(const ra_problem* p);

// Arguments of one ring-step launch (one key/value block against all local
// queries of all heads).  READ selects whether the state is read (else it
// starts empty); FINAL whether the result is normalised into out/lse (else
// the state is written back).
struct StepArgs {
  const void* q;
  const int32_t* q_pos;
  const void* k;
  const void* v;
  const int32_t* k_pos;
  const float* m_in;
  const float* l_in;
  const float* o_in;
  float* m_out;
  float* l_out;
  float* o_out;
  float* out;
  float* lse;
  unsigned long long* work;  // int64[3] {full, masked, skipped} or null
  // Per-query lower bound of the visible key positions (the first position
  // of the query's document under a document mask), or null for none.
  const int32_t* q_lo;
  int32_t n_q, n_k, h_q, h_kv, causal;
  int32_t n_qt;              // query tiles of kRowsPerGroup rows
  int32_t n_pairs;           // workgroups per head: tile t is paired with tile n_qt-1-t
  float c2;                  // scale * log2(e): scores go to base-2 units
  uint8_t head_of[kMaxHeads];  // launch-order slot -> query head (L2 locality)
  // bf16 d_k 128 step kernels: this launch covers work units (query tile
  // pair x head) [unit0, unit0 + n_units), n_units 0 meaning all of them,
  // with `groups` groups of 4 waves per workgroup (0: chosen for the launch).
  int32_t unit0, n_units, groups;
};

// All key/value blocks resident (the all-gather form): one launch folds them
// all, in order, into a register-resident state and writes out/lse.
// Ring blocks one chunk launch folds (ra_forward's chunked schedule).
constexpr int kChunkBlocks = 2;

struct MultiArgs {
  StepArgs s;  // q, q_pos, out, lse, work, sizes; s.k, s.v, s.k_pos unused
  int32_t n_blocks;
  const void* k[kMaxBlocks];
  const void* v[kMaxBlocks];
  const int32_t* k_pos[kMaxBlocks];
};

// start / stop: optional events that take the kernel's own start and end
// times (hipExtLaunchKernel); null for a plain launch.
hipError_t launch_step(const StepArgs& a, int dtype, int d_k, bool read, bool final_,
                       hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// bfloat16, d_k = 128, one group per workgroup: ma.n_blocks (1 or 2)
// consecutive ring blocks in one launch, the units of ma.s (unit0, n_units).
hipError_t launch_chunk_fast(const MultiArgs& ma, bool read, bool final_, hipStream_t stream);
// One chain of the two-chain all-gather: the blocks in ma folded by one-group
// workgroups into partial state `chain` (ma.s.m_out / l_out / o_out hold two
// states, state s at s x h_q x n_q rows in).
hipError_t launch_allgather_chain_fast(const MultiArgs& ma, int chain, hipStream_t stream);
// Merges n_states partial states (state s at m + s rows, l + s rows,
// o + s rows * d_k; bf16 d_k = 128 layout) into out and lse.
hipError_t launch_merge_states(const float* m, const float* l, const float* o, long long rows,
                               int n_states, float* out, float* lse, hipStream_t stream);
// bfloat16, d_k = 128: the 8-wave kernel with direct-to-LDS staging.
hipError_t launch_step_fast(const StepArgs& a, bool read, bool final_, hipStream_t stream,
                            hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Groups of 4 waves per workgroup the bf16 d_k 128 kernels use for a launch
// of `units` work units on the current device (1 or 2).
int fast_groups_for(long long units);
// Whether the ring runs as two chains of one-group launches (even and odd
// blocks into two states, merged at the end): one to two work units per
// compute unit.
bool fast_two_chains(long long units);
// Backward of one key/value block (bfloat16, d_k = 128): dq, dk and dv
// (fp32) each get this block's part added (dk, dv summed over the query heads
// of each key/value head).
struct BwdArgs {
  const void* q;
  const int32_t* q_pos;
  const void* k;
  const void* v;
  const int32_t* k_pos;
  const void* dout;
  const float* lse;    // [h_q][n_q], natural log, from the forward
  const float* delta;  // [h_q][n_q] = rowsum(dout * out)
  float* dq;           // [h_q][n_q][128], accumulated
  float* dk;           // [h_kv][n_k][128], accumulated
  float* dv;
  float* ws;           // [2][n_split][h_kv][n_k][128] partial sums when n_split > 1
  int32_t n_q, n_k, h_q, h_kv, causal, n_split;
  float scale, c2;
  int32_t overwrite;   // 1: dk, dv are written, not added to (0: accumulate)
  int32_t dq_write;    // 1: the per-block dq kernel writes dq instead of adding to it
};

// Splits of each head group in the dk/dv kernel, and the workspace they need.
int backward_splits(int n_k, int h_q, int h_kv);
size_t backward_ws_bytes(int n_k, int h_q, int h_kv);
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_dq(const BwdArgs& a, hipStream_t stream);

hipError_t launch_backward_dkv(const BwdArgs& a, hipStream_t stream);
// Plain per-row backward for the other supported shapes (fp32; bf16 d_k 64).
hipError_t launch_backward_generic(const BwdArgs& a, int dtype, int d_k, hipStream_t stream);
hipError_t launch_backward_delta_generic(const float* out, const void* dout, float* delta,
                                         int64_t rows, int dtype, int d_k, hipStream_t stream);
hipError_t launch_backward_delta(const float* out, const void* dout, float* delta, int64_t rows,
                                 hipStream_t stream);

// bfloat16, d_k = 128 only.
hipError_t launch_allgather_fast(const MultiArgs& ma, hipStream_t stream);
// The document-masked all-gather with the key blocks split over n_split
// workgroups per query tile (2 <= n_split <= n_blocks): partial states go to
// slots s = 0 .. n_split-1 of ma.s.m_out / l_out ([n_split][h_q * n_q]) and
// ma.s.o_out ([n_split][h_q * n_q][128]), then a merge writes out and lse.
hipError_t launch_allgather_split_fast(const MultiArgs& ma, int n_split, hipStream_t stream);
hipError_t launch_state_init(float* m, float* l, float* o, int64_t rows, int d_k,
                             hipStream_t stream);
hipError_t launch_finalize(const float* m, const float* l, const float* o, float* out,
                           float* lse, int64_t rows, int d_k, hipStream_t stream);
hipError_t launch_zero_i64(int64_t* p, int n, hipStream_t stream);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream);

}  // namespace ra
