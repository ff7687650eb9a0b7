// Host side of the C ABI declared in include/ra.h: argument checks, launch
// configuration and the ring loop of ra_forward.
//
// ra_forward follows the ring of Zero to Frontier, "distributed/context-expert",
// section "Splitting the sequence, and the one layer that objects": each step
// attends the local queries to the block held while the next block arrives,
// and no more than two blocks are held at once.  On one GPU the arrival is a
// device-to-device copy into one of two staging slots on a side stream,
// overlapped with the step running on the main stream; events keep a slot
// from being overwritten before its step has read it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/ra.h"
#include "ra_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

size_t elem_bytes(int32_t dtype) { return dtype == RA_BF16 ? 2 : 4; }

ra_status check_problem(const ra_problem* p) {
  if (!p) return RA_ERR_NULL;
  if (p->dtype != RA_BF16 && p->dtype != RA_F32) return RA_ERR_DTYPE;
  if (p->n_q < 0 || p->n_k < 0 || p->h_q < 1 || p->h_kv < 1 || p->h_q > ra::kMaxHeads)
    return RA_ERR_SHAPE;
  if (p->h_q % p->h_kv != 0) return RA_ERR_SHAPE;
  if (p->d_k != 64 && p->d_k != 128) return RA_ERR_SHAPE;
  if (p->causal != 0 && p->causal != 1) return RA_ERR_ARG;
  if (!(p->scale == 0.f || (std::isfinite(p->scale) && p->scale > 0.f))) return RA_ERR_ARG;
  // keep every element index of the largest tensor within int64 and every
  // row index within int32
  if ((int64_t)p->h_q * p->n_q > INT32_MAX || (int64_t)p->h_kv * p->n_k > INT32_MAX)
    return RA_ERR_SHAPE;
  // the kernels address one head's rows of q, k, v (and the gradients) with
  // 32-bit byte offsets and buffer sizes: each head's rows stay under 2 GiB
  const int64_t row_bytes = (int64_t)p->d_k * elem_bytes(p->dtype);
  if ((int64_t)p->n_q * row_bytes > INT32_MAX || (int64_t)p->n_k * row_bytes > INT32_MAX)
    return RA_ERR_SHAPE;
  return RA_OK;
}

float softmax_scale(const ra_problem* p) {
  return p->scale == 0.f ? 1.0f / std::sqrt((float)p->d_k) : p->scale;
}

// Launch order of query heads.  Consecutive workgroups go to different XCDs
// (8 on MI355X, each with its own L2), so slot j of every round of h_q
// workgroups lands on XCD j % 8.  Heads that share a key/value head are
// placed on the same XCD where the counts allow, so that XCD's L2 serves the
// shared block.
void head_order(const ra_problem* p, uint8_t* head_of) {
  const int hq = p->h_q, hkv = p->h_kv, g = hq / hkv;
  const int X = 8;
  bool done = false;
  if (hq % X == 0) {
    const int per = hq / X;  // query heads per XCD
    if (hkv % X == 0 || (X % hkv == 0)) {
      for (int j = 0; j < hq; ++j) {
        int x = j % X, i = j / X;  // XCD, index within the XCD
        int head;
        if (hkv % X == 0) {
          // XCD x takes KV heads x, x+X, ...; per/g of them
          int kv = x + X * (i / g);
          head = kv * g + i % g;
        } else {
          // X/hkv XCDs share each KV head
          int kv = x % hkv;
          int sub = x / hkv;  // which of the sharing XCDs
          head = kv * g + sub * per + i;
        }
        head_of[j] = (uint8_t)head;
      }
      done = true;
    }
  }
  if (!done)
    for (int j = 0; j < hq; ++j) head_of[j] = (uint8_t)j;
}

// bf16 with d_k = 128 runs the 8-wave fast kernels.
bool fast_path(const ra_problem* p) { return p->dtype == RA_BF16 && p->d_k == 128; }

// Whether ra_forward splits each ring step into two half launches, one on
// each stream.  The two chains of half launches drift apart, so each half's
// start-up, state traffic and launch gap overlap the other half's compute
// (the all-gather form has none of these costs).  The next block is staged
// on a third stream (copy_stream) meanwhile, so no half waits behind a copy.
bool split_ring(const ra_problem* p, const ra::StepArgs& a) {
  return fast_path(p) && (int64_t)a.n_pairs * a.h_q >= 2;
}

// The same split while the caller's stream is being captured into a graph:
// capturing the schedule with the third stream ended in a crash of the
// runtime's capture, so then the side stream stages the next block before
// its half, which waits for that copy.  That pays only where the copy is
// short against a step: its estimated time (K and V read and written, 8 TB/s)
// at most 5 % of the step's causal compute (half the pairs visible, 2.5
// PFLOP/s): the GQA shares (1-4 %), not the striped MHA share (15 %, 5 %
// slower split that way).
bool split_ring_two_streams(const ra_problem* p, const ra::StepArgs& a) {
  if (!split_ring(p, a)) return false;
  const double copy_s = 8.0 * p->h_kv * (double)p->n_k * p->d_k / 8e12;
  const double step_s = 2.0 * p->d_k * p->h_q * (double)p->n_q * p->n_k / 2.5e15;
  return copy_s <= 0.05 * step_s;
}

// The stream the split schedule copies blocks on: one per device, made on
// first use (default priority, not synchronising with the null stream) and
// kept until the process ends.
hipStream_t copy_stream() {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static hipStream_t streams[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [dev] {
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess) streams[dev] = s;
  });
  return streams[dev];
}

// State (m, l, o) of the per-block fallback of ra_forward_allgather.

// Key-block splits of the document-masked all-gather.  A launch of fewer than
// kSplitBelow workgroups (4 per compute unit) is split into enough of them to
// reach about kSplitTarget (8 per compute unit), at most one split per block,
// so that rows late in long documents, which see many blocks, share their
// walk among several workgroups (the kernel splits only such tiles).  A
// larger launch already spreads those walks among enough other work, and the
// partial states would only add traffic.  1 = no split (one launch, the state
// in registers).
constexpr int kSplitBelow = 1024;
constexpr int kSplitTarget = 2048;
int docs_splits(const ra_problem* p, int32_t n_cp) {
  if (!fast_path(p) || p->n_q == 0 || p->n_k == 0 || n_cp < 2) return 1;
  const int n_qt = (p->n_q + ra::kRowsPerGroup - 1) / ra::kRowsPerGroup;
  const int base = (n_qt + 1) / 2 * p->h_q;
  if (base >= kSplitBelow) return 1;
  return std::max(1, std::min<int>(n_cp, (kSplitTarget + base - 1) / base));
}

// Partial states (m, l, o) of the splits, slot after slot within each array.
struct SplitLayout {
  size_t l, o, total;
};
SplitLayout split_layout(const ra_problem* p, int n_split) {
  const size_t rows = (size_t)n_split * p->h_q * p->n_q;
  SplitLayout w;
  w.l = align_up(rows * 4);
  w.o = 2 * align_up(rows * 4);
  w.total = w.o + align_up(rows * 128 * 4);
  return w;
}

// Whether the bf16 d_k = 128 all-gather form of this problem runs as two
// chains (one to two work units per compute unit of the current device; the
// ring's rule): the even blocks and the odd blocks folded by two one-group
// launches side by side into two partial states, then merged.
bool allgather_chains(const ra_problem* p) {
  if (!fast_path(p) || p->n_q == 0 || p->n_k == 0) return false;
  const int64_t n_qt = (p->n_q + ra::kRowsPerGroup - 1) / ra::kRowsPerGroup;
  return ra::fast_two_chains((n_qt + 1) / 2 * p->h_q);
}

size_t allgather_ws_bytes(const ra_problem* p) {
  if (fast_path(p)) return allgather_chains(p) ? split_layout(p, 2).total : 0;
  const size_t rows = (size_t)p->h_q * p->n_q;
  return 2 * align_up(rows * 4) + align_up(rows * p->d_k * 4);
}

size_t docs_ws_bytes(const ra_problem* p, int32_t n_cp) {
  const int n_split = docs_splits(p, n_cp);
  if (n_split > 1) return split_layout(p, n_split).total;
  return fast_path(p) ? 0 : allgather_ws_bytes(p);  // one launch: no chains under the mask
}

ra_status fill_args(const ra_problem* p, ra::StepArgs* a) {
  std::memset(a, 0, sizeof(*a));
  a->n_q = p->n_q;
  a->n_k = p->n_k;
  a->h_q = p->h_q;
  a->h_kv = p->h_kv;
  a->causal = p->causal;
  a->n_qt = (p->n_q + ra::kRowsPerGroup - 1) / ra::kRowsPerGroup;
  a->n_pairs = (a->n_qt + 1) / 2;
  a->c2 = softmax_scale(p) * 1.4426950408889634f;
  head_order(p, a->head_of);
  return RA_OK;
}

ra_status launch(const ra_problem* p, const ra::StepArgs& a, bool read, bool final_,
                 hipStream_t s, hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
  if (a.n_qt == 0) return RA_OK;
  hipError_t e = ra::launch_step(a, p->dtype, p->d_k, read, final_, s, start, stop);
  return e == hipSuccess ? RA_OK : RA_ERR_HIP;
}

// ra_forward's workspace on the bf16 d_k = 128 path: four staging slots
// (the chunked schedule and the two-chain schedule read two blocks while the
// next two arrive) and two running states (the two chains'); elsewhere, and
// in the no-alloc form, two slots and one state.
constexpr int kChunkSlots = 4;

struct WsLayout {
  size_t m, l, o, slot[kChunkSlots], kbytes, pbytes, total;
};

// State s lives at m + s rows, l + s rows, o + s rows * d_k (floats).
WsLayout ws_layout(const ra_problem* p, int n_slots, int n_states) {
  WsLayout w;
  const size_t rows = (size_t)p->h_q * p->n_q * n_states;
  w.kbytes = (size_t)p->h_kv * p->n_k * p->d_k * elem_bytes(p->dtype);
  w.pbytes = (size_t)p->n_k * sizeof(int32_t);
  size_t off = 0;
  w.m = off;
  off = align_up(off + rows * 4);
  w.l = off;
  off = align_up(off + rows * 4);
  w.o = off;
  off = align_up(off + rows * p->d_k * 4);
  for (int s = 0; s < kChunkSlots; ++s) w.slot[s] = 0;
  for (int s = 0; s < n_slots; ++s) {
    w.slot[s] = off;  // K, then V, then positions
    off = align_up(off + w.kbytes);
    off = align_up(off + w.kbytes);
    off = align_up(off + w.pbytes);
  }
  w.total = off;
  return w;
}

// The all-gather form, with an optional per-query lower bound on the visible
// key positions (q_lo, the document start under a document mask).
ra_status allgather_impl(const ra_problem* p, int32_t n_cp, const void* q, const int32_t* q_pos,
                         const int32_t* q_lo, const void* const* k_blocks,
                         const void* const* v_blocks, const int32_t* const* k_pos_blocks,
                         void* workspace, size_t ws_bytes, float* out, float* lse, int64_t* work,
                         void* stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  if (n_cp < 1 || n_cp > ra::kMaxBlocks) return RA_ERR_SHAPE;
  if (!k_blocks || !v_blocks || !k_pos_blocks) return RA_ERR_NULL;
  if (p->n_q > 0) {
    if (!q || !q_pos || !out || !lse) return RA_ERR_NULL;
    if (!aligned16(q) || !aligned4(q_pos) || !aligned16(out) || !aligned4(lse))
      return RA_ERR_ALIGN;
  }
  if (work && !aligned8(work)) return RA_ERR_ALIGN;
  if (p->n_k > 0) {
    for (int b = 0; b < n_cp; ++b) {
      if (!k_blocks[b] || !v_blocks[b] || !k_pos_blocks[b]) return RA_ERR_NULL;
      if (!aligned16(k_blocks[b]) || !aligned16(v_blocks[b]) || !aligned4(k_pos_blocks[b]))
        return RA_ERR_ALIGN;
    }
  }
  const int n_split = q_lo ? docs_splits(p, n_cp) : 1;
  const size_t need = q_lo ? docs_ws_bytes(p, n_cp) : allgather_ws_bytes(p);
  if (need > 0) {
    if (!workspace) return RA_ERR_NULL;
    if (!aligned16(workspace)) return RA_ERR_ALIGN;
    if (ws_bytes < need) return RA_ERR_WORKSPACE;
  }

  hipStream_t s = (hipStream_t)stream;
  if (work) {
    if (ra::launch_zero_i64(work, 3, s) != hipSuccess) return RA_ERR_HIP;
  }
  if (p->n_q == 0) return RA_OK;

  ra::StepArgs a;
  fill_args(p, &a);
  a.q = q;
  a.q_pos = q_pos;
  a.q_lo = q_lo;
  a.out = out;
  a.lse = lse;
  a.work = reinterpret_cast<unsigned long long*>(work);
  if (fast_path(p)) {
    ra::MultiArgs ma;
    std::memset(&ma, 0, sizeof(ma));
    ma.s = a;
    ma.n_blocks = p->n_k > 0 ? n_cp : 0;
    for (int b = 0; b < ma.n_blocks; ++b) {
      ma.k[b] = k_blocks[b];
      ma.v[b] = v_blocks[b];
      ma.k_pos[b] = k_pos_blocks[b];
    }
    if (n_split > 1) {
      const SplitLayout w = split_layout(p, n_split);
      char* ws = (char*)workspace;
      ma.s.m_out = (float*)ws;
      ma.s.l_out = (float*)(ws + w.l);
      ma.s.o_out = (float*)(ws + w.o);
      return ra::launch_allgather_split_fast(ma, n_split, s) == hipSuccess ? RA_OK : RA_ERR_HIP;
    }
    // Two chains (see allgather_chains): the even blocks on the caller's
    // stream, the odd blocks on the library's copy stream, into the two
    // states of the workspace; then the merge on the caller's stream.  Under
    // graph capture (or if the capture state or that stream is not
    // available) one launch instead.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipStream_t cs = nullptr;
    if (!q_lo && n_cp >= 2 && allgather_chains(p) &&
        hipStreamIsCapturing(s, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone &&
        (cs = copy_stream()) != nullptr) {
      const SplitLayout w = split_layout(p, 2);
      char* ws = (char*)workspace;
      ma.s.m_out = (float*)ws;
      ma.s.l_out = (float*)(ws + w.l);
      ma.s.o_out = (float*)(ws + w.o);
      ra::MultiArgs half[2] = {ma, ma};
      for (int c = 0; c < 2; ++c) {
        half[c].n_blocks = 0;
        for (int b = c; b < n_cp; b += 2) {
          const int i = half[c].n_blocks++;
          half[c].k[i] = k_blocks[b];
          half[c].v[i] = v_blocks[b];
          half[c].k_pos[i] = k_pos_blocks[b];
        }
      }
      hipEvent_t fork = nullptr, join = nullptr;
      auto mk = [](hipEvent_t* e) {
        return hipEventCreateWithFlags(e, hipEventDisableTiming | hipEventDisableSystemFence) ==
               hipSuccess;
      };
      ra_status r = RA_ERR_HIP;
      if (mk(&fork) && mk(&join) && hipEventRecord(fork, s) == hipSuccess &&
          hipStreamWaitEvent(cs, fork, 0) == hipSuccess &&
          ra::launch_allgather_chain_fast(half[0], 0, s) == hipSuccess &&
          ra::launch_allgather_chain_fast(half[1], 1, cs) == hipSuccess &&
          hipEventRecord(join, cs) == hipSuccess && hipStreamWaitEvent(s, join, 0) == hipSuccess &&
          ra::launch_merge_states(ma.s.m_out, ma.s.l_out, ma.s.o_out,
                                  (long long)p->h_q * p->n_q, 2, out, lse, s) == hipSuccess)
        r = RA_OK;
      if (fork) (void)hipEventDestroy(fork);  // the call's status is already decided
      if (join) (void)hipEventDestroy(join);
      return r;
    }
    return ra::launch_allgather_fast(ma, s) == hipSuccess ? RA_OK : RA_ERR_HIP;
  }
  // Other shapes: one step launch per block against a state in the workspace.
  const size_t rows = (size_t)p->h_q * p->n_q;
  char* ws = (char*)workspace;
  float* m = (float*)ws;
  float* l = (float*)(ws + align_up(rows * 4));
  float* o = (float*)(ws + 2 * align_up(rows * 4));
  a.m_in = a.m_out = m;
  a.l_in = a.l_out = l;
  a.o_in = a.o_out = o;
  for (int b = 0; b < n_cp; ++b) {
    a.k = k_blocks[b];
    a.v = v_blocks[b];
    a.k_pos = k_pos_blocks[b];
    st = launch(p, a, /*read=*/b > 0, /*final=*/b == n_cp - 1, s);
    if (st != RA_OK) return st;
  }
  return RA_OK;
}

}  // namespace

extern "C" {

int32_t ra_abi_version(void) { return 1; }

int32_t ra_docs_split_span(void) { return ra::kSplitSpan; }

int32_t ra_docs_splits(const ra_problem* p, int32_t n_cp) {
  if (check_problem(p) != RA_OK || n_cp < 1 || n_cp > ra::kMaxBlocks) return 0;
  return docs_splits(p, n_cp);
}

const char* ra_status_string(ra_status s) {
  switch (s) {
    case RA_OK: return "ok";
    case RA_ERR_NULL: return "a required pointer is NULL";
    case RA_ERR_SHAPE: return "sizes out of range (h_q % h_kv, d_k in {64,128}, counts)";
    case RA_ERR_DTYPE: return "unsupported dtype (RA_BF16 or RA_F32)";
    case RA_ERR_ALIGN: return "misaligned pointer (16 B for q,k,v,o,out,workspace; 4 B positions,m,l,lse; 8 B work)";
    case RA_ERR_WORKSPACE: return "workspace too small";
    case RA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case RA_ERR_ARG: return "invalid argument (scale must be finite and > 0, causal 0 or 1; causal 1 with a document mask)";
    default: return "unknown status";
  }
}

ra_status ra_tile_shape(const ra_problem* p, int32_t* bm, int32_t* bn) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  if (!bm || !bn) return RA_ERR_NULL;
  *bm = ra::kRowsPerWave;
  *bn = ra::kKeysPerTile;
  return RA_OK;
}

ra_status ra_state_init(const ra_problem* p, float* m, float* l, float* o, void* stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  const int64_t rows = (int64_t)p->h_q * p->n_q;
  if (rows == 0) return RA_OK;
  if (!m || !l || !o) return RA_ERR_NULL;
  if (!aligned4(m) || !aligned4(l) || !aligned16(o)) return RA_ERR_ALIGN;
  hipError_t e = ra::launch_state_init(m, l, o, rows, p->d_k, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : RA_ERR_HIP;
}

ra_status ra_step(const ra_problem* p, const void* q, const int32_t* q_pos, const void* k,
                  const void* v, const int32_t* k_pos, float* m, float* l, float* o,
                  int64_t* work, void* stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  if (p->n_q == 0) return RA_OK;
  if (!q || !q_pos || !m || !l || !o) return RA_ERR_NULL;
  if (p->n_k > 0 && (!k || !v || !k_pos)) return RA_ERR_NULL;
  if (!aligned16(q) || !aligned4(q_pos) || !aligned4(m) || !aligned4(l) || !aligned16(o) ||
      (work && !aligned8(work)))
    return RA_ERR_ALIGN;
  if (p->n_k > 0 && (!aligned16(k) || !aligned16(v) || !aligned4(k_pos))) return RA_ERR_ALIGN;
  ra::StepArgs a;
  fill_args(p, &a);
  a.q = q;
  a.q_pos = q_pos;
  a.k = k;
  a.v = v;
  a.k_pos = k_pos;
  a.m_in = m;
  a.l_in = l;
  a.o_in = o;
  a.m_out = m;
  a.l_out = l;
  a.o_out = o;
  a.work = reinterpret_cast<unsigned long long*>(work);
  return launch(p, a, true, false, (hipStream_t)stream);
}

ra_status ra_finalize(const ra_problem* p, const float* m, const float* l, const float* o,
                      float* out, float* lse, void* stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  const int64_t rows = (int64_t)p->h_q * p->n_q;
  if (rows == 0) return RA_OK;
  if (!m || !l || !o || !out || !lse) return RA_ERR_NULL;
  if (!aligned4(m) || !aligned4(l) || !aligned16(o) || !aligned16(out) || !aligned4(lse))
    return RA_ERR_ALIGN;
  hipError_t e = ra::launch_finalize(m, l, o, out, lse, rows, p->d_k, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : RA_ERR_HIP;
}

size_t ra_forward_workspace_bytes(const ra_problem* p) {
  if (check_problem(p) != RA_OK) return 0;
  return fast_path(p) ? ws_layout(p, kChunkSlots, 2).total : ws_layout(p, 2, 1).total;
}

}  // extern "C"

// The no-alloc form's workspace: one running state and two staging slots (it
// runs one launch per block with its fixed events).
size_t ra::forward_noalloc_bytes(const ra_problem* p) {
  return check_problem(p) == RA_OK ? ws_layout(p, 2, 1).total : 0;
}

extern "C" {

ra_status ra_forward(const ra_problem* p, int32_t n_cp, const void* q, const int32_t* q_pos,
                     const void* const* k_blocks, const void* const* v_blocks,
                     const int32_t* const* k_pos_blocks, void* workspace, size_t ws_bytes,
                     float* out, float* lse, int64_t* work, int64_t* staged_bytes,
                     void* main_stream, void* side_stream) {
  return ra_forward_timed(p, n_cp, q, q_pos, k_blocks, v_blocks, k_pos_blocks, workspace,
                          ws_bytes, out, lse, work, staged_bytes, main_stream, side_stream,
                          nullptr, nullptr);
}

ra_status ra_forward_timed(const ra_problem* p, int32_t n_cp, const void* q, const int32_t* q_pos,
                           const void* const* k_blocks, const void* const* v_blocks,
                           const int32_t* const* k_pos_blocks, void* workspace, size_t ws_bytes,
                           float* out, float* lse, int64_t* work, int64_t* staged_bytes,
                           void* main_stream, void* side_stream, void* const* launch_events,
                           void* const* staged_events) {
  return ra::forward_ring(p, n_cp, q, q_pos, k_blocks, v_blocks, k_pos_blocks, workspace,
                          ws_bytes, out, lse, work, staged_bytes, main_stream, side_stream,
                          launch_events, staged_events, nullptr);
}

}  // extern "C"


// The ring of ra_forward.  fixed: null, or five events made by the caller
// (no timing, no system fence) that this call uses instead of creating and
// destroying its own.
ra_status ra::forward_ring(const ra_problem* p, int32_t n_cp, const void* q, const int32_t* q_pos,
                           const void* const* k_blocks, const void* const* v_blocks,
                           const int32_t* const* k_pos_blocks, void* workspace, size_t ws_bytes,
                           float* out, float* lse, int64_t* work, int64_t* staged_bytes,
                           void* main_stream, void* side_stream, void* const* launch_events,
                           void* const* staged_events, const hipEvent_t* fixed) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  if (n_cp < 1) return RA_ERR_SHAPE;
  if (!k_blocks || !v_blocks || !k_pos_blocks) return RA_ERR_NULL;
  // ra_forward's layout is what ra_forward_workspace_bytes reports; the
  // no-alloc form (fixed events: one launch per block) has two slots and one
  // state.
  const WsLayout w = fixed || !fast_path(p) ? ws_layout(p, 2, 1) : ws_layout(p, kChunkSlots, 2);
  if (p->n_q > 0) {
    if (!q || !q_pos || !out || !lse) return RA_ERR_NULL;
    if (!aligned16(q) || !aligned4(q_pos) || !aligned16(out) || !aligned4(lse))
      return RA_ERR_ALIGN;
  }
  if (work && !aligned8(work)) return RA_ERR_ALIGN;
  if (p->n_k > 0) {
    for (int b = 0; b < n_cp; ++b) {
      if (!k_blocks[b] || !v_blocks[b] || !k_pos_blocks[b]) return RA_ERR_NULL;
      if (!aligned16(k_blocks[b]) || !aligned16(v_blocks[b]) || !aligned4(k_pos_blocks[b]))
        return RA_ERR_ALIGN;
    }
  }
  if (!workspace) return RA_ERR_NULL;
  if (!aligned16(workspace)) return RA_ERR_ALIGN;
  if (ws_bytes < w.total) return RA_ERR_WORKSPACE;
  if (launch_events)
    for (int i = 0; i < 2 * n_cp; ++i)
      if (!launch_events[i]) return RA_ERR_NULL;
  if (staged_events)
    for (int i = 0; i < n_cp; ++i)
      if (!staged_events[i]) return RA_ERR_NULL;
  // Timing marks (caller-owned events); a failed record fails the call.
  auto mark = [](void* const* evs, int i, hipStream_t s) {
    return !evs || hipEventRecord((hipEvent_t)evs[i], s) == hipSuccess;
  };

  hipStream_t ms = (hipStream_t)main_stream;
  hipStream_t ss = (hipStream_t)side_stream;
  const bool use_side = ss != nullptr && ss != ms;
  char* ws = (char*)workspace;
  float* m = (float*)(ws + w.m);
  float* l = (float*)(ws + w.l);
  float* o = (float*)(ws + w.o);

  if (staged_bytes) *staged_bytes = 0;
  if (!mark(staged_events, 0, ms)) return RA_ERR_HIP;
  if (work) {
    if (ra::launch_zero_i64(work, 3, ms) != hipSuccess) return RA_ERR_HIP;
  }
  if (p->n_q == 0) {
    // nothing runs: every mark still gets recorded, so the caller can read them
    for (int b = 0; b < n_cp; ++b)
      if (!mark(launch_events, 2 * b, ms) || !mark(launch_events, 2 * b + 1, ms) ||
          (b > 0 && !mark(staged_events, b, ms)))
        return RA_ERR_HIP;
    return RA_OK;
  }

  ra::StepArgs a;
  fill_args(p, &a);
  a.q = q;
  a.q_pos = q_pos;
  a.m_in = m;
  a.l_in = l;
  a.o_in = o;
  a.m_out = m;
  a.l_out = l;
  a.o_out = o;
  a.out = out;
  a.lse = lse;
  a.work = reinterpret_cast<unsigned long long*>(work);

  // Events: slot s staged (side -> main), slot s consumed (main -> side), the
  // caller's prior work on main (main -> side) before the first copy, and
  // the side stream's last half launch (side -> main) in the split schedule.
  hipEvent_t ev_staged[kChunkSlots] = {}, ev_used[kChunkSlots] = {}, ev_used2[kChunkSlots] = {},
            ev_start = nullptr, ev_join = nullptr;
  ra_status result = RA_OK;
  int64_t staged = 0;
  // Split schedule: each step's launch is two halves of the work units, one
  // on each stream (see split_ring); caller-made events or timing marks keep
  // the one-launch schedule.
  // Under graph capture (or if the capture state cannot be read) the split
  // stages on the side stream (split_ring_two_streams); otherwise on the
  // copy stream cs.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  const bool capturing = hipStreamIsCapturing(ms, &cap) != hipSuccess ||
                         cap != hipStreamCaptureStatusNone;
  hipStream_t cs = nullptr;
  const bool split_ok = use_side && n_cp > 1 && fixed == nullptr && launch_events == nullptr &&
                        staged_events == nullptr;
  const bool three = split_ok && !capturing && split_ring(p, a) && (cs = copy_stream()) != nullptr;
  const bool split = three || (split_ok && split_ring_two_streams(p, a));
  const int split_groups = split ? ra::fast_groups_for((int64_t)a.n_pairs * a.h_q) : 0;
  // Chunked schedule: with the copy stream, one-group workgroups and a
  // four-slot workspace, launches fold two blocks each ([0], [1, 2], [3, 4],
  // ...) with the state in registers between them; block b >= 1 is staged
  // into slot (b - 1) % 4.
  const bool chunked = three && split_groups == 1 && n_cp >= 3;
  // Two chains: with the copy stream, where one chain of one-group launches
  // would leave compute units with a single workgroup (one to two work units
  // per compute unit), even blocks fold into state 0 on the main stream and
  // odd blocks into state 1 on the side stream, one full-grid one-group
  // launch per block, and a merge of the two states writes out and lse.
  // Rounding differs from one chain; tile counts do not.
  const bool chains = three && ra::fast_two_chains((int64_t)a.n_pairs * a.h_q);
  const int n_slots = chunked || chains ? kChunkSlots : 2;
  auto slot_of = [&](int b) { return n_slots == kChunkSlots ? (b - 1) % kChunkSlots : b & 1; };
  // The events only order work between two streams of this device; the copy
  // kernels' completion and the step kernels' launch carry their own memory
  // fences, so the events skip the system-scope fence (a cache writeback and
  // invalidate that cost several microseconds between steps).
  auto mk = [](hipEvent_t* e) {
    return hipEventCreateWithFlags(e, hipEventDisableTiming | hipEventDisableSystemFence) ==
           hipSuccess;
  };
  // Copies block b (b >= 1) into its slot on stream dst, after the launch
  // that last read that slot (block b - n_slots) is done, and marks it staged.
  auto stage = [&](int b, hipStream_t dst) {
    const int s = slot_of(b);
    char* slot = ws + w.slot[s];
    if (use_side && b - n_slots >= 1 &&
        (hipStreamWaitEvent(dst, ev_used[s], 0) != hipSuccess ||
         (three && !chains && hipStreamWaitEvent(dst, ev_used2[s], 0) != hipSuccess)))
      return false;
    if (w.kbytes &&
        (hipMemcpyAsync(slot, k_blocks[b], w.kbytes, hipMemcpyDeviceToDevice, dst) != hipSuccess ||
         hipMemcpyAsync(slot + align_up(w.kbytes), v_blocks[b], w.kbytes, hipMemcpyDeviceToDevice,
                        dst) != hipSuccess ||
         hipMemcpyAsync(slot + 2 * align_up(w.kbytes), k_pos_blocks[b], w.pbytes,
                        hipMemcpyDeviceToDevice, dst) != hipSuccess))
      return false;
    staged += 2 * (int64_t)w.kbytes;
    if (!mark(staged_events, b, dst)) return false;
    return !use_side || hipEventRecord(ev_staged[s], dst) == hipSuccess;
  };
  if (use_side && n_cp > 1) {
    if (fixed) {
      ev_start = fixed[0];
      ev_staged[0] = fixed[1];
      ev_staged[1] = fixed[2];
      ev_used[0] = fixed[3];
      ev_used[1] = fixed[4];
    } else {
      bool ok = mk(&ev_start) && (!split || mk(&ev_join));
      for (int i = 0; ok && i < n_slots; ++i)
        ok = mk(&ev_staged[i]) && mk(&ev_used[i]) && (!three || mk(&ev_used2[i]));
      if (!ok) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
    }
    if (hipEventRecord(ev_start, ms) != hipSuccess ||
        hipStreamWaitEvent(ss, ev_start, 0) != hipSuccess ||
        (three && hipStreamWaitEvent(cs, ev_start, 0) != hipSuccess)) {
      result = RA_ERR_HIP;
      goto cleanup;
    }
  }

  if (chunked) {
    // launch c folds blocks c0 .. c0 + nb - 1: [0], [1, 2], [3, 4], ...
    const int n_launch = 1 + n_cp / 2;
    const int total = a.n_pairs * a.h_q, half = total / 2;
    auto blocks_of = [&](int c, int& c0, int& nb) {
      c0 = c == 0 ? 0 : 2 * c - 1;
      nb = c == 0 ? 1 : std::min(2, n_cp - c0);
    };
    for (int c = 0; c < n_launch; ++c) {
      int c0, nb;
      blocks_of(c, c0, nb);
      const bool first = c == 0, last = c == n_launch - 1;
      ra::MultiArgs ma;
      ma.s = a;
      ma.n_blocks = nb;
      for (int i = 0; i < nb; ++i) {
        const int b = c0 + i;
        if (b == 0) {
          ma.k[i] = k_blocks[0];
          ma.v[i] = v_blocks[0];
          ma.k_pos[i] = k_pos_blocks[0];
          continue;
        }
        // both halves wait for the block's copy
        const int sl = slot_of(b);
        if (hipStreamWaitEvent(ms, ev_staged[sl], 0) != hipSuccess ||
            hipStreamWaitEvent(ss, ev_staged[sl], 0) != hipSuccess) {
          result = RA_ERR_HIP;
          goto cleanup;
        }
        char* slot = ws + w.slot[sl];
        ma.k[i] = slot;
        ma.v[i] = slot + align_up(w.kbytes);
        ma.k_pos[i] = (const int32_t*)(slot + 2 * align_up(w.kbytes));
      }
      ra::MultiArgs ha = ma, hb = ma;
      ha.s.unit0 = 0;
      ha.s.n_units = half;
      hb.s.unit0 = half;
      hb.s.n_units = total - half;
      if (ra::launch_chunk_fast(ha, !first, last, ms) != hipSuccess) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
      // the next launch's blocks go to their slots on the copy stream
      if (c + 1 < n_launch) {
        int n0, nn;
        blocks_of(c + 1, n0, nn);
        for (int i = 0; i < nn; ++i)
          if (!stage(n0 + i, cs)) {
            result = RA_ERR_HIP;
            goto cleanup;
          }
      }
      if (ra::launch_chunk_fast(hb, !first, last, ss) != hipSuccess) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
      // the slots of this launch's blocks are free once both halves are done
      for (int i = 0; i < nb; ++i) {
        const int b = c0 + i;
        if (b >= 1 && b + n_slots < n_cp &&
            (hipEventRecord(ev_used[slot_of(b)], ms) != hipSuccess ||
             hipEventRecord(ev_used2[slot_of(b)], ss) != hipSuccess)) {
          result = RA_ERR_HIP;
          goto cleanup;
        }
      }
    }
  } else if (chains) {
    // block b on the main stream into state 0 (b even) or on the side stream
    // into state 1 (b odd); block b + 2 staged on the copy stream meanwhile
    const size_t rows = (size_t)p->h_q * p->n_q;
    ra::StepArgs c = a;
    c.groups = 1;
    if (!stage(1, cs)) {
      result = RA_ERR_HIP;
      goto cleanup;
    }
    for (int b = 0; b < n_cp; ++b) {
      hipStream_t st = (b & 1) ? ss : ms;
      const size_t sidx = b & 1;
      c.m_in = c.m_out = m + sidx * rows;
      c.l_in = c.l_out = l + sidx * rows;
      c.o_in = c.o_out = o + sidx * rows * p->d_k;
      if (b == 0) {
        c.k = k_blocks[0];
        c.v = v_blocks[0];
        c.k_pos = k_pos_blocks[0];
      } else {
        const int sl = slot_of(b);
        if (hipStreamWaitEvent(st, ev_staged[sl], 0) != hipSuccess) {
          result = RA_ERR_HIP;
          goto cleanup;
        }
        char* slot = ws + w.slot[sl];
        c.k = slot;
        c.v = slot + align_up(w.kbytes);
        c.k_pos = (const int32_t*)(slot + 2 * align_up(w.kbytes));
      }
      result = launch(p, c, /*read=*/b >= 2, /*final=*/false, st);
      if (result != RA_OK) goto cleanup;
      // the slot is free for block b + 4 once this launch is done
      if (b >= 1 && b + n_slots < n_cp && hipEventRecord(ev_used[slot_of(b)], st) != hipSuccess) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
      if (b + 2 < n_cp && !stage(b + 2, cs)) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
    }
  } else
  for (int b = 0; b < n_cp; ++b) {
    const bool first = b == 0, last = b == n_cp - 1;
    if (first) {
      a.k = k_blocks[0];
      a.v = v_blocks[0];
      a.k_pos = k_pos_blocks[0];
    } else {
      // the split schedule staged block b during step b - 1
      if (!split && !stage(b, use_side ? ss : ms)) { result = RA_ERR_HIP; goto cleanup; }
      if (use_side && hipStreamWaitEvent(ms, ev_staged[b & 1], 0) != hipSuccess) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
      char* slot = ws + w.slot[b & 1];
      a.k = slot;
      a.v = slot + align_up(w.kbytes);
      a.k_pos = (const int32_t*)(slot + 2 * align_up(w.kbytes));
    }
    if (split) {
      // first half on the main stream, second half on the side stream (which
      // also waits for this block's copy), block b + 1 staged on the copy
      // stream meanwhile (or on the side stream before its half)
      if (three && !first && hipStreamWaitEvent(ss, ev_staged[b & 1], 0) != hipSuccess) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
      const int total = a.n_pairs * a.h_q, half = total / 2;
      ra::StepArgs ha = a, hb = a;
      ha.unit0 = 0;
      ha.n_units = half;
      hb.unit0 = half;
      hb.n_units = total - half;
      ha.groups = hb.groups = split_groups;
      result = launch(p, ha, /*read=*/!first, /*final=*/last, ms);
      if (result != RA_OK) goto cleanup;
      if (b + 1 < n_cp && !stage(b + 1, three ? cs : ss)) { result = RA_ERR_HIP; goto cleanup; }
      result = launch(p, hb, /*read=*/!first, /*final=*/last, ss);
      if (result != RA_OK) goto cleanup;
    } else {
      // with timing, the kernel's own start and end times go to the events
      result = launch(p, a, /*read=*/!first, /*final=*/last, ms,
                      launch_events ? (hipEvent_t)launch_events[2 * b] : nullptr,
                      launch_events ? (hipEvent_t)launch_events[2 * b + 1] : nullptr);
      if (result != RA_OK) goto cleanup;
    }
    if (use_side && !first && b + 2 < n_cp) {
      // slot b & 1 is free for block b + 2 once this step is done: its
      // main-stream part, and with the copy stream its side-stream part
      // (otherwise that precedes the copy on the side stream)
      if (hipEventRecord(ev_used[b & 1], ms) != hipSuccess ||
          (three && hipEventRecord(ev_used2[b & 1], ss) != hipSuccess)) {
        result = RA_ERR_HIP;
        goto cleanup;
      }
    }
  }
  if (split && (hipEventRecord(ev_join, ss) != hipSuccess ||
                hipStreamWaitEvent(ms, ev_join, 0) != hipSuccess)) {
    result = RA_ERR_HIP;
    goto cleanup;
  }
  // the two chains' states merged into out and lse (the online-softmax
  // combination of two partial states)
  if (chains && ra::launch_merge_states(m, l, o, (long long)p->h_q * p->n_q, 2, out, lse, ms) !=
                    hipSuccess) {
    result = RA_ERR_HIP;
    goto cleanup;
  }
  if (staged_bytes) *staged_bytes = staged;

cleanup:
  if (!fixed)
    for (hipEvent_t e : {ev_start, ev_join, ev_staged[0], ev_staged[1], ev_staged[2], ev_staged[3],
                         ev_used[0], ev_used[1], ev_used[2], ev_used[3], ev_used2[0], ev_used2[1],
                         ev_used2[2], ev_used2[3]})
      if (e) (void)hipEventDestroy(e);  // the call's status is already decided
  return result;
}

extern "C" {

ra_status ra_backward_prep(const ra_problem* p, const float* out, const void* dout,
                           float* delta, void* stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  const int64_t rows = (int64_t)p->h_q * p->n_q;
  if (rows == 0) return RA_OK;
  if (!out || !dout || !delta) return RA_ERR_NULL;
  if (!aligned16(out) || !aligned16(dout) || !aligned4(delta)) return RA_ERR_ALIGN;
  hipError_t e = fast_path(p)
                     ? ra::launch_backward_delta(out, dout, delta, rows, (hipStream_t)stream)
                     : ra::launch_backward_delta_generic(out, dout, delta, rows, p->dtype, p->d_k,
                                                         (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : RA_ERR_HIP;
}

size_t ra_backward_workspace_bytes(const ra_problem* p) {
  if (check_problem(p) != RA_OK || !fast_path(p)) return 0;
  return ra::backward_ws_bytes(p->n_k, p->h_q, p->h_kv);
}

ra_status ra_backward_step(const ra_problem* p, const void* q, const int32_t* q_pos,
                           const void* k, const void* v, const int32_t* k_pos, const void* dout,
                           const float* lse, const float* delta, float* dq, float* dk, float* dv,
                           void* workspace, size_t workspace_bytes, void* stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  const bool fast = fast_path(p);
  const size_t need = fast ? ra::backward_ws_bytes(p->n_k, p->h_q, p->h_kv) : 0;
  if (need > 0 && p->n_k > 0) {
    if (!workspace) return RA_ERR_NULL;
    if (workspace_bytes < need) return RA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return RA_ERR_ALIGN;
  }
  if (p->n_q > 0 && (!q || !q_pos || !dout || !lse || !delta || !dq)) return RA_ERR_NULL;
  if (p->n_k > 0 && (!k || !v || !k_pos || !dk || !dv)) return RA_ERR_NULL;
  if (p->n_q > 0 && (!aligned16(q) || !aligned4(q_pos) || !aligned16(dout) || !aligned4(lse) ||
                     !aligned4(delta) || !aligned16(dq)))
    return RA_ERR_ALIGN;
  if (p->n_k > 0 && (!aligned16(k) || !aligned16(v) || !aligned4(k_pos) || !aligned16(dk) ||
                     !aligned16(dv)))
    return RA_ERR_ALIGN;
  if (p->n_q == 0 && p->n_k == 0) return RA_OK;
  ra::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.q_pos = q_pos;
  a.k = k;
  a.v = v;
  a.k_pos = k_pos;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.n_q = p->n_q;
  a.n_k = p->n_k;
  a.h_q = p->h_q;
  a.h_kv = p->h_kv;
  a.causal = p->causal;
  a.n_split = fast ? ra::backward_splits(p->n_k, p->h_q, p->h_kv) : 1;
  a.ws = (float*)workspace;
  a.scale = softmax_scale(p);
  a.c2 = a.scale * 1.4426950408889634f;
  const hipError_t e =
      fast ? ra::launch_backward(a, (hipStream_t)stream)
           : ra::launch_backward_generic(a, p->dtype, p->d_k, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : RA_ERR_HIP;
}

namespace {
// Workspace of ra_backward_share: delta, then the head-group partial sums the
// dk/dv kernel writes (shared by the blocks, whose dk/dv steps are ordered).
struct BwdShareLayout {
  size_t delta, part, total;
};
BwdShareLayout bwd_share_layout(const ra_problem* p) {
  BwdShareLayout w;
  w.delta = 0;
  w.part = align_up((size_t)p->h_q * p->n_q * sizeof(float));
  const size_t part = fast_path(p) ? ra::backward_ws_bytes(p->n_k, p->h_q, p->h_kv) : 0;
  w.total = w.part + align_up(part);
  return w;
}
}  // namespace

size_t ra_backward_share_workspace_bytes(const ra_problem* p) {
  if (check_problem(p) != RA_OK) return 0;
  return bwd_share_layout(p).total;
}

ra_status ra_backward_share(const ra_problem* p, int32_t n_cp, const void* q,
                            const int32_t* q_pos, const void* const* k_blocks,
                            const void* const* v_blocks, const int32_t* const* k_pos_blocks,
                            const float* out, const float* lse, const void* dout, float* dq,
                            float* const* dk_blocks, float* const* dv_blocks, void* workspace,
                            size_t ws_bytes, void* main_stream, void* side_stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  if (n_cp < 1) return RA_ERR_SHAPE;
  if (!k_blocks || !v_blocks || !k_pos_blocks || !dk_blocks || !dv_blocks) return RA_ERR_NULL;
  if (p->n_q > 0) {
    if (!q || !q_pos || !out || !lse || !dout || !dq) return RA_ERR_NULL;
    if (!aligned16(q) || !aligned4(q_pos) || !aligned16(out) || !aligned4(lse) ||
        !aligned16(dout) || !aligned16(dq))
      return RA_ERR_ALIGN;
  }
  if (p->n_k > 0) {
    for (int b = 0; b < n_cp; ++b) {
      if (!k_blocks[b] || !v_blocks[b] || !k_pos_blocks[b] || !dk_blocks[b] || !dv_blocks[b])
        return RA_ERR_NULL;
      if (!aligned16(k_blocks[b]) || !aligned16(v_blocks[b]) || !aligned4(k_pos_blocks[b]) ||
          !aligned16(dk_blocks[b]) || !aligned16(dv_blocks[b]))
        return RA_ERR_ALIGN;
    }
  }
  const BwdShareLayout w = bwd_share_layout(p);
  if (w.total > 0) {
    if (!workspace) return RA_ERR_NULL;
    if (!aligned16(workspace)) return RA_ERR_ALIGN;
    if (ws_bytes < w.total) return RA_ERR_WORKSPACE;
  }

  const bool fast = fast_path(p);
  hipStream_t ms = (hipStream_t)main_stream;
  hipStream_t ss = (hipStream_t)side_stream;
  const bool use_side = fast && ss != nullptr && ss != ms;
  hipStream_t ks = use_side ? ss : ms;  // dk/dv work
  char* ws = (char*)workspace;
  float* delta = (float*)(ws + w.delta);
  const int64_t rows = (int64_t)p->h_q * p->n_q;
  const int64_t kv_elems = (int64_t)p->h_kv * p->n_k * p->d_k;

  ra::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.q_pos = q_pos;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.n_q = p->n_q;
  a.n_k = p->n_k;
  a.h_q = p->h_q;
  a.h_kv = p->h_kv;
  a.causal = p->causal;
  a.n_split = fast ? ra::backward_splits(p->n_k, p->h_q, p->h_kv) : 1;
  a.ws = (float*)(ws + w.part);
  a.scale = softmax_scale(p);
  a.c2 = a.scale * 1.4426950408889634f;

  hipEvent_t ev_ready = nullptr, ev_done = nullptr;
  ra_status result = RA_OK;
  auto hip = [&](hipError_t e) {
    if (e != hipSuccess && result == RA_OK) result = RA_ERR_HIP;
    return e == hipSuccess;
  };
  auto mk = [](hipEvent_t* e) {
    return hipEventCreateWithFlags(e, hipEventDisableTiming | hipEventDisableSystemFence) ==
           hipSuccess;
  };
  // bf16 d 128: dk and dv are written, not accumulated, and the first
  // block's dq kernel writes dq, so nothing is zeroed first; the other
  // shapes accumulate onto zeros.
  a.overwrite = fast ? 1 : 0;
  // delta first (main stream); the dk/dv steps wait for it
  if (rows > 0) {
    if (!fast && !hip(ra::launch_zero_f32(dq, rows * p->d_k, ms))) goto cleanup;
    if (!hip(fast ? ra::launch_backward_delta(out, dout, delta, rows, ms)
                  : ra::launch_backward_delta_generic(out, dout, delta, rows, p->dtype, p->d_k,
                                                      ms)))
      goto cleanup;
  }
  if (use_side) {
    if (!mk(&ev_ready) || !mk(&ev_done)) {
      result = RA_ERR_HIP;
      goto cleanup;
    }
    if (!hip(hipEventRecord(ev_ready, ms)) || !hip(hipStreamWaitEvent(ss, ev_ready, 0)))
      goto cleanup;
  }
  for (int b = 0; b < n_cp; ++b) {
    a.k = k_blocks[b];
    a.v = v_blocks[b];
    a.k_pos = k_pos_blocks[b];
    a.dk = dk_blocks[b];
    a.dv = dv_blocks[b];
    if (!fast && p->n_k > 0) {
      if (!hip(ra::launch_zero_f32(a.dk, kv_elems, ks)) ||
          !hip(ra::launch_zero_f32(a.dv, kv_elems, ks)))
        goto cleanup;
    }
    if (fast) {
      // the first block's dq kernel writes dq, the later ones add to it
      a.dq_write = b == 0 ? 1 : 0;
      if (p->n_q > 0 && !hip(ra::launch_backward_dq(a, ms))) goto cleanup;
      if (!hip(ra::launch_backward_dkv(a, ks))) goto cleanup;
    } else if (p->n_q > 0 || p->n_k > 0) {
      if (!hip(ra::launch_backward_generic(a, p->dtype, p->d_k, ms))) goto cleanup;
    }
  }
  if (use_side) {
    if (!hip(hipEventRecord(ev_done, ss)) || !hip(hipStreamWaitEvent(ms, ev_done, 0)))
      goto cleanup;
  }

cleanup:
  for (hipEvent_t e : {ev_ready, ev_done})
    if (e) (void)hipEventDestroy(e);  // the call's status is already decided
  return result;
}

size_t ra_forward_allgather_workspace_bytes(const ra_problem* p) {
  if (check_problem(p) != RA_OK) return 0;
  return allgather_ws_bytes(p);
}

ra_status ra_forward_allgather(const ra_problem* p, int32_t n_cp, const void* q,
                               const int32_t* q_pos, const void* const* k_blocks,
                               const void* const* v_blocks, const int32_t* const* k_pos_blocks,
                               void* workspace, size_t ws_bytes, float* out, float* lse,
                               int64_t* work, void* stream) {
  return allgather_impl(p, n_cp, q, q_pos, nullptr, k_blocks, v_blocks, k_pos_blocks, workspace,
                        ws_bytes, out, lse, work, stream);
}

size_t ra_forward_allgather_docs_workspace_bytes(const ra_problem* p, int32_t n_cp) {
  if (check_problem(p) != RA_OK || n_cp < 1 || n_cp > ra::kMaxBlocks) return 0;
  return docs_ws_bytes(p, n_cp);
}

ra_status ra_forward_allgather_docs(const ra_problem* p, int32_t n_cp, const void* q,
                                    const int32_t* q_pos, const int32_t* q_doc_start,
                                    const void* const* k_blocks, const void* const* v_blocks,
                                    const int32_t* const* k_pos_blocks, void* workspace,
                                    size_t ws_bytes, float* out, float* lse, void* stream) {
  ra_status st = check_problem(p);
  if (st != RA_OK) return st;
  if (p->causal != 1) return RA_ERR_ARG;
  if (p->n_q > 0) {
    if (!q_doc_start) return RA_ERR_NULL;
    if (!aligned4(q_doc_start)) return RA_ERR_ALIGN;
  }
  return allgather_impl(p, n_cp, q, q_pos, q_doc_start, k_blocks, v_blocks, k_pos_blocks,
                        workspace, ws_bytes, out, lse, nullptr, stream);
}

}  // extern "C"
