/*
 * ringattn.h -- C ABI of one device's share of a Ring Attention forward pass
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed ("Ring Attention" (aarnphm.xyz), the recurrence for S, m,
 * z, y and O): device `rank` (u) holds its query block Q^(u) and sees the P
 * key/value blocks in ring order b(u, s) = (u - s) mod P, s = 0 .. P-1.  Each
 * visit forms S = Q K^T / sqrt(d_h), folds it into the running per-row
 * (m, z, y) with the rescale factor exp(m_old - m_new), and after the last
 * visit O = y / z.  The log-sum-exp LSE = m + ln z (natural log) is written
 * beside O, the per-row statistics the transformer-math page (aicassindra.com),
 * section "The backward pass costs a second ring", says are kept.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, on the
 *    current HIP device, 16-byte aligned, densely packed row-major.
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *    stream).  Every call is asynchronous on `stream`: it is ordered after the
 *    work already on `stream`, and work enqueued later on `stream` sees the
 *    results.  Inputs must stay alive and unmodified until then.
 *  - Batch is 1.  Query head h reads key/value head h / (Hq / Hkv).
 *  - Return value: RINGATTN_OK or an error code.  Argument errors are reported
 *    before any HIP call is made and nothing is enqueued.  Nothing throws or
 *    aborts across this ABI.  ringattn_last_error() gives a message for the
 *    last failure on the calling thread.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RINGATTN_OK = 0,
  RINGATTN_EINVAL = 1,       /* bad shape, null pointer, misalignment, out-of-range argument */
  RINGATTN_EUNSUPPORTED = 2, /* valid but not implemented (e.g. d_h not in {64, 128}) */
  RINGATTN_EHIP = 3          /* the HIP runtime reported an error (message has the detail) */
};

enum { RINGATTN_LAYOUT_CONTIGUOUS = 0, RINGATTN_LAYOUT_STRIPED = 1, RINGATTN_LAYOUT_ZIGZAG = 2 };

/* How the next visit's key/value block reaches its slot (ringattn_set_hop_mode). */
enum { RINGATTN_HOP_FUSED = 0, RINGATTN_HOP_SERIAL = 1, RINGATTN_HOP_STREAMS = 2 };

/*
 * ringattn_forward -- rank `rank`'s share of the ring, bf16 in and out.
 *
 * Shard layout (layout): the sequence of N tokens is split into P shards of
 * b = N / P tokens.  CONTIGUOUS: shard r holds tokens r*b .. r*b+b-1 (the
 * transformer-math page, "The mechanism, compressed").  STRIPED: token t lives
 * on shard t mod P, so local row j of shard r is token j*P + r ("Ring
 * Attention" (aarnphm.xyz): striped ownership balances causal work).  ZIGZAG:
 * the sequence is cut into 2P chunks of c = b/2 tokens and shard r holds chunk
 * r followed by chunk 2P-1-r, so local row j < c is token r*c + j and row
 * j >= c is token (2P-1-r)*c + j - c ("Ring Attention" (darshanfofadiya.com),
 * 4.8.3: one early and one late block per GPU gives every GPU the same causal
 * work).
 * Causal (causal = 1): a query attends to keys at GLOBAL token positions <= its
 * own ("Ring Attention" (darshanfofadiya.com), 4.8 and 4.8.1).
 *
 *  q    [b, Hq, d_h]        bf16, rank's query rows in local order (read only)
 *  k, v [P, b, Hkv, d_h]    bf16, every shard, shard-major, each in local row
 *                           order: what the ring would deliver (read only).
 *                           Shard `rank` is the device's own block.
 *  out  [b, Hq, d_h]        bf16, O (written)
 *  lse  [Hq, b]             fp32, natural-log LSE (written), may be NULL
 *  N, P, rank               N % P == 0 (N % 2P == 0 for ZIGZAG), N >= P >= 1,
 *                           0 <= rank < P
 *  Hq, Hkv                  Hq % Hkv == 0
 *  d_h                      64 or 128
 *  causal                   0 or 1
 *  layout                   RINGATTN_LAYOUT_CONTIGUOUS, _STRIPED or _ZIGZAG
 *  Limits: b <= 2^28, Hq * b <= 2^25 and Hkv <= 65536 (the kernels index
 *  rows in 32 bits); a larger shape returns RINGATTN_EUNSUPPORTED.
 *
 * The library allocates its workspace (two key/value slots and the fp32 running
 * state) stream-ordered on `stream` and frees it the same way.  The block for
 * step s+1 is copied into the free slot while step s computes, by default by
 * the step launch's own workgroups after their tiles (ringattn_set_hop_mode):
 * the one-GPU stand-in for the ring hop.
 */
int ringattn_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t N, int P, int rank, int Hq, int Hkv, int d_h,
                     int causal, int layout, void* stream);

/* ringattn_forward_f32 -- identical to ringattn_forward with fp32 q, k, v and
 * out; every quantity is computed in fp32. */
int ringattn_forward_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                         int64_t N, int P, int rank, int Hq, int Hkv, int d_h,
                         int causal, int layout, void* stream);

/*
 * ringattn_backward -- rank `rank`'s share of the backward ring (the
 * transformer-math page (aicassindra.com), "The backward pass costs a second
 * ring"): the P key/value blocks visit again in the forward's ring order; for
 * each visit the scores are rebuilt from the saved LSE rather than stored,
 *   P = exp(S - LSE),  D = rowsum(dO * O),  dS = P * (dP - D),  dP = dO V^T,
 * dQ of the rank's rows collects dS K / sqrt(d_h) over all visits, and the
 * visiting block's gradient accumulators collect this rank's contribution
 * dK_r += dS^T Q / sqrt(d_h), dV_r += P^T dO, as they would while rotating
 * with the block.  Gradients are of L = sum(dO * O) for the O of
 * ringattn_forward with the same shapes, mask and layout.
 *
 *  q, out, dout [b, Hq, d_h]     bf16: the rank's query rows, the forward's O
 *                                and the upstream gradient (read only)
 *  lse          [Hq, b]          fp32, the forward's LSE (natural log)
 *  k, v         [P, b, Hkv, d_h] bf16, every shard as for ringattn_forward
 *  dq           [b, Hq, d_h]     fp32, dL/dQ of the rank's rows (written)
 *  dk, dv       [P, b, Hkv, d_h] fp32, ADDED TO: this rank's contribution to
 *                                every shard's dL/dK and dL/dV (blocks the
 *                                rank never sees get nothing).  Zero them
 *                                before the first rank; after all P ranks
 *                                they hold the full gradients.
 *  N, P, rank, Hq, Hkv, d_h, causal, layout as for ringattn_forward, with
 *  the same limits.  Every pointer is required and 16-byte aligned.
 *
 * The library allocates its workspace (the query rows' packed tiles and two
 * packed key/value slots) stream-ordered on `stream`; the slot of visit s+1 is
 * packed while visit s computes, by default by the dK/dV workgroups of visit
 * s's launch before their own work (ringattn_set_hop_mode).  Each visit is
 * one launch whose workgroups compute either dK, dV or dQ.
 */
int ringattn_backward(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      int64_t N, int P, int rank, int Hq, int Hkv, int d_h,
                      int causal, int layout, void* stream);

/*
 * ringattn_merge -- combine `nparts` partial (m, z, y) triples of the same
 * rows with one rescale-and-add (the transformer-math page, "The ring is a
 * prefill algorithm": each shard returns a partial (m, l, o) and one small
 * reduction combines them).  m* = max_i m_i, w_i = exp(m_i - m*),
 * O = sum_i w_i y_i / sum_i w_i z_i, LSE = m* + ln sum_i w_i z_i.
 *
 *  m, z  [nparts, Hq, rows]       fp32; m in natural-log units, z >= 0
 *  y     [nparts, rows, Hq, d_h]  fp32, unnormalised
 *  out   [rows, Hq, d_h]          out_dtype: 0 = bf16, 1 = fp32 (written)
 *  lse   [Hq, rows]               fp32 (written), may be NULL
 *  A partial with m = -inf, z = 0 contributes nothing; a row whose partials
 *  are all empty gets O = 0 and LSE = -inf.  nparts >= 1, rows >= 0, Hq >= 1,
 *  d_h in {64, 128}; rows * Hq <= 2^30, else RINGATTN_EUNSUPPORTED.  rows = 0
 *  is valid and enqueues nothing.
 */
int ringattn_merge(const float* m, const float* z, const float* y, int nparts,
                   int64_t rows, int Hq, int d_h, void* out, int out_dtype,
                   float* lse, void* stream);

/*
 * ringattn_decode_partial -- pass-Q decode on one device: the new query rows
 * meet the device's resident key/value shard, which stays in place, and give
 * a partial (m, z, y) triple; ringattn_merge combines the P devices' partials
 * into O and LSE (the transformer-math page (aicassindra.com), "The ring is a
 * prefill algorithm": keep the cache sharded and stationary, broadcast the
 * query, combine P partial (m, l, o) with one small reduction; "Ring
 * Attention" (darshanfofadiya.com) 4.9.4.4, the pass-Q variant).  The new
 * tokens follow every cached key, so no key of the shard is masked:
 *   m = max_j S_j,  z = sum_j e^{S_j - m},  y = sum_j e^{S_j - m} v_j,
 *   S_j = q . k_j / sqrt(d_h), over the shard's n_keys keys.
 *
 *  q        [n_q, Hq, d_h]      bf16, the new tokens' query rows (read only)
 *  k, v     [n_keys, Hkv, d_h]  bf16, the resident shard (read only); may be
 *                               NULL when n_keys == 0
 *  m, z     [Hq, n_q]           fp32 (written): m in natural-log units
 *  y        [n_q, Hq, d_h]      fp32, unnormalised (written)
 *  n_q >= 1, n_keys >= 0, Hq % Hkv == 0, d_h in {64, 128}.  q, k, v and y
 *  must be 16-byte aligned, m and z 4-byte aligned.  Limits: Hq * n_q <= 2^30,
 *  (Hq / Hkv) * n_q <= 16 * 65535 and ceil(n_keys / 256) <= 2^30, else
 *  RINGATTN_EUNSUPPORTED.
 *
 * These are exactly one part of ringattn_merge's inputs: pointing m, z, y at
 * part p of arrays [P, Hq, n_q] and [P, n_q, Hq, d_h] and then calling
 * ringattn_merge(..., nparts = P, rows = n_q, ...) gives attention of the new
 * tokens over every shard.  An empty shard (n_keys = 0) gives m = -inf, z = 0,
 * y = 0, which the merge ignores.  The library takes a workspace of
 * ceil(n_keys / 256) * Hq * n_q * (d_h + 2) floats stream-ordered on `stream`.
 */
int ringattn_decode_partial(const void* q, const void* k, const void* v, int n_q,
                            int64_t n_keys, int Hq, int Hkv, int d_h,
                            float* m, float* z, float* y, void* stream);

/*
 * ringattn_decode_partial_noalloc -- ringattn_decode_partial for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, same kernels and
 * bit-identical results, but the chunk partials live in a static device
 * buffer of the library instead of a stream-ordered allocation.  The call
 * makes no hipMalloc, hipFree or other allocating call.
 *
 *  Limit: the call needs 2 * round_up(4 * ceil(n_keys / 256) * Hq * n_q, 256)
 *  + 4 * ceil(n_keys / 256) * Hq * n_q * d_h bytes of scratch, at most 32 MiB
 *  (e.g. 31,250 keys x 64/8 heads x d 128 takes 4.1 MB; one 131,072-key shard
 *  x 4/1 heads 1.1 MB).  A larger call returns RINGATTN_EUNSUPPORTED before
 *  any HIP call.
 *  The buffer: one per device, 32 MiB, held by every device the library runs
 *  on until the process ends.  Every call on a device uses the same buffer:
 *  calls that overlap on one device (other streams, other threads) race and
 *  give wrong results; calls on one stream, or ordered by events, are safe.
 *  Nothing in it needs to start at zero: each call writes every partial it
 *  reads.  The first call on a device looks up the buffer's device address.
 *  These calls are not timed by ringattn_timing_enable.
 */
int ringattn_decode_partial_noalloc(const void* q, const void* k, const void* v, int n_q,
                                    int64_t n_keys, int Hq, int Hkv, int d_h,
                                    float* m, float* z, float* y, void* stream);

/* Static string for a status code. */
const char* ringattn_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* ringattn_last_error(void);

/*
 * Kernel timing for measurement.  While enabled (enable = 1) every step kernel
 * that ringattn_forward / ringattn_forward_f32 launches, every merge kernel and
 * the kernels of every ringattn_decode_partial call are bracketed by a pair of
 * HIP events on the stream they run on.  ringattn_timing_collect() waits for
 * the recorded step and merge events, returns the summed duration (ms) and
 * count of the step kernels and of the merge kernels since the last collect,
 * and releases those events.  Returns a status code.
 */
int ringattn_timing_enable(int enable);
int ringattn_timing_collect(double* step_ms, int64_t* step_launches,
                            double* merge_ms, int64_t* merge_launches);

/* Same for the visit launches of ringattn_backward (dK/dV and dQ of a visit
 * in one launch): summed duration (ms) and number of visits. */
int ringattn_timing_collect_backward(double* step_ms, int64_t* step_launches);

/* Same for ringattn_decode_partial calls: summed duration (ms) of the decode
 * kernels of each call (chunk and combine kernels together) and the number of
 * calls since the last collect of decode timings. */
int ringattn_timing_collect_decode(double* decode_ms, int64_t* decode_calls);

/*
 * Diagnostics of the bf16 step kernel's rescale schedule.  Its fast pipeline
 * keeps one fixed softmax reference per row; a workgroup whose probabilities
 * would leave the safe range against it (a later score far above the
 * reference: "Ring Attention" (aarnphm.xyz), the rescale factor
 * exp(m_old - m_new) of the recurrence for m, z, y) starts over on the exact
 * path with the running maximum.  This call waits for all work on the current
 * device, then writes the number of step-kernel workgroups that did so since
 * the previous call (redone) and how many of those had been folding the
 * carried running state in late (redone_late_fold), and clears both counts.
 * Either pointer may be NULL.  The counts are per device and shared by every
 * caller on it.
 */
int ringattn_redo_count(int64_t* redone, int64_t* redone_late_fold);

/*
 * How the ring's hop (the next visit's key/value block copied into the free
 * slot of the double buffer; "Ring Attention" (darshanfofadiya.com), 4.5
 * "Communication-Computation Overlap") is scheduled, for every later call on
 * any device:
 *   RINGATTN_HOP_FUSED   (default) the step launch of visit i also copies the
 *                        block of visit i+1, in its workgroups' tails, so the
 *                        copy overlaps the step inside one launch and no
 *                        cross-stream event is needed (ringattn_backward:
 *                        the dK/dV workgroups of visit i's launch copy the
 *                        block of visit i+1 before their own work).  ringattn_forward_f32,
 *                        whose step kernel has no copy, uses
 *                        RINGATTN_HOP_SERIAL instead;
 *   RINGATTN_HOP_SERIAL  a copy kernel on the caller's stream between steps;
 *   RINGATTN_HOP_STREAMS a copy kernel on the library's second stream beside
 *                        the next step, ordered by events.
 * Results are bit-identical in every mode.  Returns RINGATTN_EINVAL for
 * another value.
 */
int ringattn_set_hop_mode(int mode);

/*
 * Earlier form of ringattn_set_hop_mode: serial = 1 selects
 * RINGATTN_HOP_SERIAL, 0 RINGATTN_HOP_FUSED.
 */
int ringattn_set_serial_hops(int serial);

/* Library version, e.g. "ringattn 0.1.0 gfx950". */
const char* ringattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
