/*
 * ra.h -- C ABI of the MI355X (gfx950) ring-attention rank-share library.
 *
 * One context-parallel rank holds n_q queries at explicit global token
 * positions and meets every key/value block of the sequence once, one block
 * per ring step (Zero to Frontier, "distributed/context-expert", section
 * "Splitting the sequence, and the one layer that objects": each step the
 * GPU attends its queries to the block it holds while passing that block to
 * its right neighbour and receiving the next from its left).  For every query
 * it keeps the online-softmax state -- running maximum m of the scores,
 * running sum l of their exponentials, unnormalised weighted value sum O --
 * and rescales the old totals whenever a block brings a larger score (same
 * section; also the "Context Parallelism (CP)" concept page, "Key math / How
 * it works").  After the last block, out = O / l and lse = m + ln l.
 *
 * Conventions for every entry point:
 *  - Pointers named q, k, v, *_pos, m, l, o, out, lse, work and workspace are
 *    DEVICE pointers, allocated and owned by the caller; the library keeps
 *    none of them past the call.  Arrays of block pointers passed to
 *    ra_forward are HOST arrays of device pointers.  staged_bytes is a host
 *    pointer.
 *  - Layouts are row-major with d_k fastest:  q[h_q][n_q][d_k],
 *    k, v[h_kv][n_k][d_k], m, l[h_q][n_q], o, out[h_q][n_q][d_k], lse[h_q][n_q].
 *    Element type of q, k, v: bfloat16 (RA_BF16) or float (RA_F32).  State,
 *    out and lse are float.  q, k, v, o, out and workspace must be 16-byte
 *    aligned; positions, m, l and lse 4-byte; work 8-byte.
 *  - q_pos[n_q] and k_pos[n_k] are int32 global positions in [0, 2^31-2],
 *    strictly increasing within each array (true of the contiguous, zigzag
 *    and striped layouts).  Key j is visible to query i iff
 *    k_pos[j] <= q_pos[i] when causal, always otherwise (and, through
 *    ra_forward_allgather_docs only, not before the query's document start).
 *    Positions that do not increase give unspecified values but never an
 *    out-of-bounds access.
 *  - Query head h reads key/value head h / (h_q / h_kv).
 *  - State (m, l, O): m is the running maximum of the scores s = scale * q.k
 *    (natural-log units) over the visible keys seen so far, l = sum exp(s - m)
 *    and O = sum exp(s - m) v over the same keys.  A row that has seen no
 *    visible key has m = -inf, l = 0, O = 0.
 *  - Calls are asynchronous on the given HIP stream (passed as void*, a
 *    hipStream_t; NULL is the default stream).  Arguments are checked on the
 *    host first: on an error nothing is enqueued and no output is touched.
 *    RA_ERR_HIP reports a failed launch or enqueue; a fault inside a kernel
 *    surfaces at the caller's next synchronisation.
 *  - The library holds no mutable global state: concurrent calls on
 *    different streams are safe when their output buffers do not overlap.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ra_status;
enum {
  RA_OK = 0,
  RA_ERR_NULL = -1,      /* a required pointer is NULL */
  RA_ERR_SHAPE = -2,     /* sizes out of range, h_q % h_kv != 0, d_k not 64/128, n_cp < 1 */
  RA_ERR_DTYPE = -3,     /* dtype not RA_BF16 / RA_F32 */
  RA_ERR_ALIGN = -4,     /* a pointer breaks the alignment rules above */
  RA_ERR_WORKSPACE = -5, /* workspace smaller than ra_forward_workspace_bytes() */
  RA_ERR_HIP = -6,       /* a HIP runtime call or launch failed */
  RA_ERR_ARG = -7        /* scale not finite and > 0 (or 0 for the default); causal not 1
                            with a document mask */
};

enum { RA_BF16 = 0, RA_F32 = 1 };

typedef struct ra_problem {
  int32_t n_q;    /* queries on this rank, >= 0 */
  int32_t n_k;    /* keys per key/value block, >= 0 (all blocks equal); one head's
                     rows of q (n_q) and of a block (n_k) each under 2 GiB, i.e.
                     n * d_k * element size <= 2^31 - 1 (RA_ERR_SHAPE otherwise) */
  int32_t h_q;    /* query heads, 1..256 */
  int32_t h_kv;   /* key/value heads, h_q % h_kv == 0 */
  int32_t d_k;    /* head width: 64 or 128 */
  int32_t dtype;  /* RA_BF16 or RA_F32: element type of q, k, v */
  int32_t causal; /* 1: key j visible to query i iff k_pos[j] <= q_pos[i]; 0: all */
  float scale;    /* softmax scale; 0 selects 1/sqrt(d_k) */
} ra_problem;

/* Fill the state with the empty row: m = -inf, l = 0, o = 0. */
ra_status ra_state_init(const ra_problem* p, float* m, float* l, float* o, void* stream);

/*
 * One ring step: fold the attention of q against one key/value block into the
 * state (m, l, o) in place.  Exactly the online-softmax rescale of Zero to
 * Frontier, "distributed/context-expert", section "Splitting the sequence,
 * and the one layer that objects" (and the "Context Parallelism (CP)" concept
 * page, "Key math / How it works"): the new running max, the old totals times
 * exp(old max - new max), plus this block's terms against the new max.
 * Rows that see no key of the block are left untouched.
 * work: optional device int64[3] that gets += {full, masked, skipped} tile
 * counts of this block (query tiles x key tiles of ra_tile_shape(), counted
 * for head 0 only since the classes do not depend on the head); NULL skips it.
 */
ra_status ra_step(const ra_problem* p, const void* q, const int32_t* q_pos,
                  const void* k, const void* v, const int32_t* k_pos,
                  float* m, float* l, float* o, int64_t* work, void* stream);

/* Normalise after the last block (same section of Zero to Frontier: the
 * output is the weighted sum divided by the exp-sum; the log-sum-exp is the
 * running max plus the log of the exp-sum): out = o / l, lse = m + ln l; a row
 * with l == 0 gives out = 0, lse = -inf. */
ra_status ra_finalize(const ra_problem* p, const float* m, const float* l, const float* o,
                      float* out, float* lse, void* stream);

/* Bytes of device workspace ra_forward needs: the running state and the
 * staging slots for incoming key/value blocks.  In general one state and two
 * slots (the ring's block being computed and the one arriving); for bf16
 * with d_k = 128 two states and four slots, for the schedules that read two
 * blocks at a time while the next two arrive (see ra_forward). */
size_t ra_forward_workspace_bytes(const ra_problem* p);

/*
 * The whole rank share: n_cp ring steps then normalisation.
 * k_blocks, v_blocks, k_pos_blocks: HOST arrays of n_cp device pointers, in
 * ring order; entry 0 is the rank's own block (used in place), and block b
 * is the one received at step b.  Each block b >= 1 is copied into a staging
 * slot of the workspace while earlier blocks compute -- a one-GPU stand-in
 * for the ring receive -- with events so a slot is never overwritten before
 * the launch that reads it is done.  Schedules:
 *  - side_stream NULL or equal to main_stream: everything on main_stream;
 *  - otherwise, shapes other than bf16 with d_k = 128: one launch per step
 *    on main_stream, copies on side_stream;
 *  - bf16, d_k = 128, copies on a stream the library creates once per
 *    device, and by the number of work units (query-tile pairs x query
 *    heads) against the device's compute units:
 *    - at least two per compute unit: each launch's work split in two
 *      halves, one on main_stream and one on side_stream; launches after the
 *      first take two blocks each (n_cp >= 3, the state kept in registers
 *      between them: the same bits as one launch per block);
 *    - one to two: two chains, the even blocks folded into one running state
 *      on main_stream and the odd blocks into a second one on side_stream,
 *      merged into out and lse at the end (the online-softmax combination of
 *      two partial states; rounding differs from one chain, tile counts do
 *      not);
 *    - fewer: each launch split in two halves as above, one block each.
 *    While main_stream is being captured into a graph: one block per launch
 *    and the copies on side_stream (split only where the copy is short
 *    against a step).
 * out, lse: results.  work: optional device int64[3], zeroed and then filled
 * with the tile counts summed over all steps.  staged_bytes: optional host
 * pointer, receives the key/value bytes copied into staging slots
 * ((n_cp - 1) blocks of 2 * h_kv * n_k * d_k elements).
 * The workspace contents after the call are unspecified.  Work on
 * main_stream after the call sees the results; nothing is left pending on
 * side_stream that touches caller memory.
 */
ra_status ra_forward(const ra_problem* p, int32_t n_cp, const void* q, const int32_t* q_pos,
                     const void* const* k_blocks, const void* const* v_blocks,
                     const int32_t* const* k_pos_blocks, void* workspace, size_t ws_bytes,
                     float* out, float* lse, int64_t* work, int64_t* staged_bytes,
                     void* main_stream, void* side_stream);

/*
 * ra_forward with timing marks, for measuring the ring on one GPU: the
 * per-step kernel time and how much of the next block's staging shows
 * between steps (Zero to Frontier, "distributed/context-expert", section
 * "When the ring hides its communication": the exchange for the next step
 * runs while this step computes and costs nothing when it finishes first).
 * Arguments and behaviour are those of ra_forward, plus:
 *  launch_events: NULL, or a HOST array of 2 * n_cp hipEvent_t handles (as
 *    void*) created by the caller with timing enabled.  Entries 2b and 2b+1
 *    take the start and end times of step b's kernel itself (the launch
 *    goes through hipExtLaunchKernel with them), so their difference is that
 *    kernel's duration and the time from 2b-1 to 2b the gap between steps.
 *  staged_events: NULL, or a HOST array of n_cp such handles.  Entry 0 is
 *    recorded on main_stream before any work of the call; entry b >= 1 on the
 *    stream that copies block b, right after its copies.
 * The events stay owned by the caller; read them after synchronising.  With
 * both arrays NULL the call is ra_forward.
 */
ra_status ra_forward_timed(const ra_problem* p, int32_t n_cp, const void* q, const int32_t* q_pos,
                           const void* const* k_blocks, const void* const* v_blocks,
                           const int32_t* const* k_pos_blocks, void* workspace, size_t ws_bytes,
                           float* out, float* lse, int64_t* work, int64_t* staged_bytes,
                           void* main_stream, void* side_stream, void* const* launch_events,
                           void* const* staged_events);

/*
 * ra_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  Arguments and results are those of ra_forward.
 * It runs one launch per block (the one-block schedules of ra_forward), so
 * it needs one running state (fp32 m and l of h_q x n_q rows, o of
 * h_q x n_q x d_k) and two staging slots (a block's K, V and positions),
 * which live in a fixed array of RA_NOALLOC_MAX_BYTES that every device the
 * library runs on holds from the library's load until the process ends; the
 * first call on a device takes that array's address and creates five
 * ordering events (once), and no call allocates device memory.  A problem
 * whose state and two slots (16-byte aligned each) exceed
 * RA_NOALLOC_MAX_BYTES is refused with RA_ERR_WORKSPACE before any work.  Nothing in the array needs to start at zero (every step writes
 * what it later reads), but all calls on one device share it: calls that
 * overlap in time on one device race and give unspecified results.
 */
#define RA_NOALLOC_MAX_BYTES ((size_t)256 << 20)
ra_status ra_forward_noalloc(const ra_problem* p, int32_t n_cp, const void* q,
                             const int32_t* q_pos, const void* const* k_blocks,
                             const void* const* v_blocks, const int32_t* const* k_pos_blocks,
                             float* out, float* lse, int64_t* work, int64_t* staged_bytes,
                             void* main_stream, void* side_stream);

/* Bytes of device workspace ra_forward_allgather needs.  bfloat16 with
 * d_k = 128: 0 (the state stays in registers), except where the launch has
 * one to two work units (query-tile pairs x query heads) per compute unit of
 * the current device: two partial states (m, l, o) for the two chains (see
 * ra_forward_allgather).  Other shapes: the running state (m, l, o). */
size_t ra_forward_allgather_workspace_bytes(const ra_problem* p);

/*
 * The rank share in its all-gather form (Zero to Frontier,
 * "distributed/context-expert": section "Splitting the sequence, and the one
 * layer that objects" gathers every key/value block before one attention pass
 * over the local queries, and "What context parallelism communicates"
 * contrasts it with the ring: same bytes, all moved first, full K and V
 * held).  All n_cp blocks are resident: k_blocks, v_blocks, k_pos_blocks are
 * HOST arrays of n_cp device pointers, 1 <= n_cp <= 64; the result does not
 * depend on their order beyond rounding.  bfloat16 with d_k = 128 runs one
 * launch that folds every block into a register-resident state and writes
 * out/lse; with one to two work units per compute unit and n_cp >= 2 it runs
 * two such launches side by side instead, the even blocks on stream and the
 * odd blocks on a stream the library creates once per device, each into a
 * partial state in the workspace, merged into out/lse on stream (one launch
 * while stream is being captured into a graph).  Other shapes run one step
 * launch per block against the state kept in the workspace.  The workspace
 * holds ra_forward_allgather_workspace_bytes(p) bytes (it may be NULL when
 * that is 0).  out, lse and work as in ra_forward.  Asynchronous on stream:
 * work after the call on stream sees the results.
 */
ra_status ra_forward_allgather(const ra_problem* p, int32_t n_cp, const void* q,
                               const int32_t* q_pos, const void* const* k_blocks,
                               const void* const* v_blocks, const int32_t* const* k_pos_blocks,
                               void* workspace, size_t ws_bytes, float* out, float* lse,
                               int64_t* work, void* stream);

/* Bytes of device workspace ra_forward_allgather_docs needs for n_cp blocks
 * (0 for an invalid problem or n_cp).  bfloat16 with d_k = 128 splits the
 * key blocks over several workgroups per query tile when the launch would
 * otherwise be small, and keeps their partial states (m, l, o) here; other
 * shapes need ra_forward_allgather_workspace_bytes(p). */
size_t ra_forward_allgather_docs_workspace_bytes(const ra_problem* p, int32_t n_cp);

/*
 * The all-gather form under a document mask (packed sequences: Zero to
 * Frontier, "distributed/context-expert", section "Splitting the sequence,
 * and the one layer that objects", gives easy support of arbitrary masks such
 * as document masks as one reason to gather the keys and values first).  As
 * ra_forward_allgather, plus q_doc_start: a DEVICE int32[n_q] holding, for
 * each query, the first global position of the document it belongs to.  Key
 * j is visible to query i iff q_doc_start[i] <= k_pos[j] <= q_pos[i], which
 * for documents packed one after another is "the same document and not
 * later".  Requirements: p->causal == 1 (RA_ERR_ARG otherwise);
 * q_doc_start[i] <= q_pos[i] and non-decreasing in i (true for packed
 * documents, since q_pos increases); 4-byte aligned (RA_ERR_ALIGN); not
 * NULL when n_q > 0 (RA_ERR_NULL).  Values breaking the ordering give
 * unspecified results but no out-of-bounds access.  A query whose document
 * has no key among the blocks gets out = 0 and lse = -inf.  No tile counters
 * (the causal work counts of ra_forward describe the causal mask alone).
 * workspace: ra_forward_allgather_docs_workspace_bytes(p, n_cp) bytes of
 * device memory, 16-byte aligned (RA_ERR_WORKSPACE if ws_bytes is smaller,
 * RA_ERR_NULL if it is needed and NULL); its contents after the call are
 * unspecified.  With split key blocks the partial states are combined in a
 * second launch, so results agree with ra_forward_allgather on a single
 * document to rounding, not bit for bit.  Asynchronous on stream; calls
 * sharing a workspace must be ordered; the caller owns every buffer.
 */
ra_status ra_forward_allgather_docs(const ra_problem* p, int32_t n_cp, const void* q,
                                    const int32_t* q_pos, const int32_t* q_doc_start,
                                    const void* const* k_blocks, const void* const* v_blocks,
                                    const int32_t* const* k_pos_blocks, void* workspace,
                                    size_t ws_bytes, float* out, float* lse, void* stream);

/*
 * Backward of the rank share (Zero to Frontier, "distributed/context-expert",
 * section "Splitting the sequence, and the one layer that objects": the
 * backward mirrors the forward; each GPU computes, from its own queries, the
 * gradients of every key/value block it sees, returned to the block's owner
 * as a second circulating block in the ring or by a reduce-scatter in the
 * all-gather form).  Every shape the forward takes: bfloat16 with d_k = 128
 * runs on MFMA kernels (p and ds rounded to bfloat16 as MFMA operands); fp32
 * and bfloat16 with d_k = 64 run on plain per-row kernels in fp32 (correct,
 * not tuned).  With s = scale q.k over visible pairs and the
 * forward's lse (natural log, over all blocks): p = exp(s - lse),
 * delta = rowsum(dout * out), ds = p (dout.v - delta).
 *
 * ra_backward_prep: delta[h_q][n_q] (fp32) from out[h_q][n_q][d_k] (fp32, the
 * forward's output) and dout[h_q][n_q][d_k] (the inputs' dtype).
 * ra_backward_step: one key/value block.  All three gradients are
 * ACCUMULATED: dq[h_q][n_q][d_k] (fp32) += scale * sum_j ds k_j (zero it
 * before the first block); dk, dv[h_kv][n_k][d_k] (fp32) += this rank's part
 * of the block's gradients, dk = scale * sum_i ds q_i and dv = sum_i p dout_i,
 * summed over the query heads that read each key/value head (pass zeros for a
 * block's own gradients, or the block's travelling gradients received from
 * the ring neighbour).  q, k, v, dout 16-byte aligned, as the
 * forward's; dq, dk, dv 16-byte aligned.  When few key/value heads leave the
 * dk/dv grid small, the query heads of each group are split across
 * workgroups: each split writes partial sums into the caller's workspace
 * (ra_backward_workspace_bytes(p) bytes, 16-byte aligned, device memory,
 * contents unspecified after the call) and they are added in a fixed order,
 * so results do not depend on scheduling.  A call that needs no workspace
 * (the size is 0) accepts NULL.  Returns RA_ERR_WORKSPACE when it is too
 * small.  Asynchronous on stream; calls sharing a workspace must be ordered.
 */
ra_status ra_backward_prep(const ra_problem* p, const float* out, const void* dout,
                           float* delta, void* stream);
size_t ra_backward_workspace_bytes(const ra_problem* p);
ra_status ra_backward_step(const ra_problem* p, const void* q, const int32_t* q_pos,
                           const void* k, const void* v, const int32_t* k_pos, const void* dout,
                           const float* lse, const float* delta, float* dq, float* dk, float* dv,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of the whole rank share in one call, every block resident (the
 * all-gather form of Zero to Frontier, "distributed/context-expert", section
 * "Splitting the sequence, and the one layer that objects": this rank's
 * dK/dV contributions are then reduce-scattered to the blocks' owners).
 * Block b is k_blocks[b], v_blocks[b], k_pos_blocks[b] as in ra_forward.
 * Writes (OVERWRITES) dq[h_q][n_q][d_k] and, per block, dk_blocks[b] and
 * dv_blocks[b][h_kv][n_k][d_k] (fp32) with this rank's gradients, from the
 * forward's out (fp32) and lse and the output gradient dout (inputs' dtype).
 * Workspace: ra_backward_share_workspace_bytes(p) bytes, 16-byte aligned,
 * device memory (delta and the head-group partial sums; contents unspecified
 * after the call); NULL is accepted when the size is 0.  With side_stream
 * non-NULL and different from main_stream (bfloat16 with d_k = 128), the
 * dk/dv kernels run on side_stream beside the dq kernels on main_stream;
 * side_stream first waits for main_stream's prior work and main_stream ends
 * waiting for side_stream, so the results are complete in main_stream order.
 * Asynchronous; the same shapes and error codes as ra_backward_step.
 */
size_t ra_backward_share_workspace_bytes(const ra_problem* p);
ra_status ra_backward_share(const ra_problem* p, int32_t n_cp, const void* q,
                            const int32_t* q_pos, const void* const* k_blocks,
                            const void* const* v_blocks, const int32_t* const* k_pos_blocks,
                            const float* out, const float* lse, const void* dout, float* dq,
                            float* const* dk_blocks, float* const* dv_blocks, void* workspace,
                            size_t ws_bytes, void* main_stream, void* side_stream);

/* Query-tile rows (bm) and key-tile columns (bn) the tile counters use.  The
 * classes follow the causal picture of Zero to Frontier, "distributed/
 * context-expert", section "The causal mask unbalances the sequence": a tile
 * whose keys all precede its queries is full, one that straddles the diagonal
 * is masked, one wholly after it is skipped. */
ra_status ra_tile_shape(const ra_problem* p, int32_t* bm, int32_t* bn);

/* Static description of a status code. */
const char* ra_status_string(ra_status s);

/* Matrix-pipe calibration (measurement support, not a step of the pages'
 * method): n_workgroups workgroups of 8 waves (two per SIMD) each issue
 * 4 * iters v_mfma_f32_32x32x16_bf16 on independent accumulators, with no
 * memory traffic, and write one float per workgroup to sink (device,
 * n_workgroups floats, 4-byte aligned).  Each workgroup performs
 * 8 * 4 * iters * 32768 FLOPs; timing the call on its stream gives the bf16
 * MFMA rate the device sustains under full matrix-pipe load, the ceiling
 * against which the attention kernels' rates are also read.  RA_ERR_SHAPE
 * for n_workgroups or iters below 1. */
ra_status ra_mfma_ceiling(int32_t n_workgroups, int32_t iters, float* sink, void* stream);

/* ABI version of this header (bumped on any incompatible change). */
int32_t ra_abi_version(void);

/* The document-masked all-gather (ra_forward_allgather_docs) splits a long
 * key walk over several workgroups when its launch alone would leave compute
 * units idle: ra_docs_splits() gives the number of splits for this problem
 * and n_cp (1 = one workgroup per query tile pair; 0 for a bad problem or
 * n_cp outside 1..64), and a tile of 128 query rows is split only when its
 * last row's position lies more than ra_docs_split_span() positions past its
 * first row's document start.  Host-only; no device work. */
int32_t ra_docs_split_span(void);
int32_t ra_docs_splits(const ra_problem* p, int32_t n_cp);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
