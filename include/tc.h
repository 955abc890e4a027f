/*
 * tc.h -- C ABI of the Tensor Cache (TC) layer on AMD Instinct MI355X (gfx950).
 *
 * The layer is the one described in "Tensor Cache: Eviction-conditioned
 * Associative Memory for Transformers" (Swain, Han, Weidele, Martino,
 * Torralba, 2026):
 *   L1 (Section 3.1, Eq. 1): exact causal softmax attention of q_t over the W
 *       most recent keys/values, i.e. keys max(0, t-W+1) .. t.
 *   L2 (Section 3.2, Figure 2 step 3): a per-head D x D matrix A, A_0 = 0,
 *       written only when a pair leaves the window:
 *       A_t = lambda_h * A_{t-1} + eta_h * k_{t-W} (outer) v_{t-W}   (t >= W)
 *       A[a][c] accumulates k[a]*v[c].
 *   Read + fuse (Figure 2 step 5): m_t = q_t A_t (no normaliser),
 *       y_t = y_local,t + sigmoid(g_h) * m_t.
 *   Prefill/training computes A with the exact parallel weighted-sum scan of
 *   the abstract (equal to per-token writes up to float rounding), never the
 *   chunk-mean shortcut.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous.
 *     The caller owns every buffer; the library allocates nothing.
 *   - q, k, v, y, dy, dq, dk, dv and the rings share the element type
 *     `dtype` (TC_F32 or TC_BF16).  lambda, eta, gate, A, lse and the
 *     parameter gradients are float32.  pos is int64.
 *   - Arithmetic is float32 (bf16 operands on the matrix cores, float32
 *     accumulation, float32 softmax and state); bf16 outputs are rounded to
 *     nearest even.
 *   - Supported head dims: D in {16, 32, 64, 128}; anything else returns
 *     TC_ERR_UNSUPPORTED.  Any T >= 1, W >= 1, C >= 1.
 *   - Device-side preconditions that are NOT checked (checking would need a
 *     synchronisation): lambda in [0,1], eta >= 0, finite inputs, pos >= 0.
 *     NaN/Inf inputs propagate to the outputs.
 *   - All argument checks run on the host before any HIP call; a failed check
 *     returns TC_ERR_INVALID_ARGUMENT / TC_ERR_UNSUPPORTED / TC_ERR_WORKSPACE
 *     and writes nothing.  A failed kernel launch returns TC_ERR_HIP.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Nothing synchronises except tc_forward_status, which
 *     is a query.  The library's only global mutable state is a call counter
 *     (it makes each forward call's flag value unique) and a per-device cache
 *     of how many forward workgroups the device holds at once; both are
 *     updated atomically, so calls on different streams or host threads with
 *     disjoint buffers may run concurrently.  Results are deterministic (no
 *     floating-point atomics).
 */
#ifndef TC_H_
#define TC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TC_OK = 0,
  TC_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, aliased output */
  TC_ERR_UNSUPPORTED = 2,      /* head dim or dtype not built */
  TC_ERR_WORKSPACE = 3,        /* workspace missing or too small */
  TC_ERR_HIP = 4,              /* a HIP launch (or the status query's copy) failed */
  TC_ERR_STATE_EXCHANGE = 5    /* tc_forward_status: a wait for another workgroup's
                                  segment state ran out; the affected rows and the
                                  final state were written as NaN */
} tc_status_t;

typedef enum { TC_F32 = 0, TC_BF16 = 1 } tc_dtype_t;

/* Prefill / training shapes.  scale <= 0 selects 1/sqrt(D) (the standard
 * scaled dot product; the pages do not state the scale).  C is the chunk
 * length of the scan.  The exact weighted-sum scan (tc_forward, the
 * backward, the continuation) gives results that do not depend on it (only
 * float rounding does): its kernels read the state per query block (128 rows
 * for bf16 with D <= 64, else 64) and advance it in 64-token steps whatever
 * C is.  C matters to tc_forward_chunk_mean, the chunk-mean shortcut. */
typedef struct {
  int32_t B, H, T, D, W, C;
  float scale;
  int32_t dtype; /* tc_dtype_t */
} tc_shape_t;

/* Decode shapes: S independent streams of H heads, ring of W slots. */
typedef struct {
  int32_t S, H, D, W;
  float scale;
  int32_t dtype; /* tc_dtype_t */
} tc_decode_shape_t;

/* Bytes of device workspace tc_forward / tc_backward need for `shape`
 * (0 if the shape is invalid).  The workspace holds the eviction-state
 * checkpoints of the scan, for the forward one 64-bit flag per segment and
 * one 64-bit status word per workgroup and, for the backward, per-row and
 * per-block partial sums.  Its contents on entry are ignored: a forward call
 * waits only for a flag value of its own (a per-process random salt combined
 * with a call count), which stale contents do not hold. */
size_t tc_forward_workspace_size(const tc_shape_t* shape);
size_t tc_backward_workspace_size(const tc_shape_t* shape);

/*
 * tc_forward -- prefill / training forward (Section 3.1 Eq. 1, Section 3.2,
 * Figure 2; the scan of the abstract).
 *   q, k, v  [B,H,T,D] dtype, post-RoPE (RoPE, if any, is applied by the
 *            caller before the keys enter the window, Section 3.1).
 *   lambda, eta, gate [H] float32: per-head decay, write rate, gate logit.
 *   y        [B,H,T,D] dtype, out.
 *   A_final  [B,H,D,D] float32, out, nullable: A after step T-1 (the state a
 *            decode continuing at position T starts from).
 *   lse      [B,H,T] float32, out, nullable: natural-log softmax normaliser
 *            of the scaled window scores (needed by tc_backward).
 *   ws       device workspace of at least tc_forward_workspace_size bytes;
 *            calls that overlap in time must not share one.
 * Outputs must not overlap the inputs or each other.  With one 128-row block
 * per segment the workgroups of the launch hand segment states to each other
 * through flags in the workspace; a wait is bounded (environment variable
 * TC_FORWARD_MAX_POLLS, default 65536 polls) and one that runs out yields
 * NaN in the affected rows instead of a stale state, and leaves a mark in
 * the workspace that tc_forward_status reports.  (The waits are only for
 * workgroups dispatched earlier, which wait for nothing later, so they end
 * well inside the bound.)  A call made while its stream is being captured
 * into a HIP graph takes the path without flags (a separate state pass), so
 * graph replays stay correct.
 */
tc_status_t tc_forward(const tc_shape_t* shape, const void* q, const void* k, const void* v,
                       const float* lambda, const float* eta, const float* gate, void* y,
                       float* A_final, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * tc_forward_chunk_mean -- the chunk-mean shortcut that the exact scan
 * replaces (abstract; Section 1, contributions; Section 2, training
 * considerations): the eviction stream in chunks of C pairs, each chunk
 * written once as its mean pair, A <- lambda A + eta (kbar outer vbar).
 * It exists to measure what the shortcut costs and how far it lands from
 * the exact scan.  Read between writes (the pages do not say; the chunked
 * scan's inter-chunk state): a query at step t >= W whose evicted token t-W
 * lies in chunk n = (t-W)/C reads the memory after chunks 0 .. n-1; earlier
 * queries read nothing.  A_final (nullable) is the memory after every
 * complete chunk; L1, y, lse and the arguments are as for tc_forward, with
 * the same workspace (tc_forward_workspace_size).
 * Built for bf16 with D in {16, 32, 64}, C in {64, 128} and W a multiple of
 * C; other shapes return TC_ERR_UNSUPPORTED.
 */
tc_status_t tc_forward_chunk_mean(const tc_shape_t* shape, const void* q, const void* k, const void* v,
                                  const float* lambda, const float* eta, const float* gate, void* y,
                                  float* A_final, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * tc_forward_delta -- the layer with the delta-rule write that Figure 2
 * (step 3) names as the optional alternative to the outer product.  The pages
 * give no formula; reading (Widrow-Hoff error correction, Section 2): the
 * evicted pair first reads the memory and only the prediction error is
 * written, u = v_old - k_old A (A before the write), A <- lambda A +
 * eta (k_old outer u).  L1, the read m_t = q_t A_t, the gate, y and lse are
 * as for tc_forward; A_final (nullable) is the memory after step T-1.
 * Computed in chunks of 64 evictions (a triangular solve per chunk, a walk
 * over the chunks per (b,h)) in float32; C is not used.
 *   ws   device workspace of at least tc_forward_delta_workspace_size(shape)
 *        bytes (the chunks' float32 intermediates and the memory read).
 * Every shape tc_forward accepts; errors as for tc_forward.
 */
size_t tc_forward_delta_workspace_size(const tc_shape_t* shape);
tc_status_t tc_forward_delta(const tc_shape_t* shape, const void* q, const void* k, const void* v,
                             const float* lambda, const float* eta, const float* gate, void* y, float* A_final,
                             float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * tc_forward_noalloc -- tc_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and results.  Instead of a caller's workspace it uses a static
 * device array of 32 MiB that the library holds on each GPU it runs on until
 * the process ends; it calls no hipMalloc, hipFree or other allocating
 * routine.  The array belongs to the current device (the stream must be one
 * of its streams); its address is looked up once per device on the first
 * call there.
 *   Limit: the shape's forward workspace (tc_forward_workspace_size) must be
 *   at most 32 MiB (33554432 bytes), else TC_ERR_WORKSPACE and nothing runs;
 *   e.g. B=8 H=8 T=1024 D=64 needs 9.4 MB and B=1 H=12 T=32768 D=64 25.4 MB.
 *   Every call on one GPU shares its array and leaves its contents there (no
 *   part of it needs clearing: stale flags never match a later call's flag
 *   value).  Calls that overlap in time on one GPU (other streams, other
 *   host threads) race on it and must be serialised by the caller.
 *   tc_forward_status cannot be queried for these calls; a flag wait that
 *   ran out shows only as NaN rows.
 * Other errors as for tc_forward; TC_ERR_HIP also when the array's device
 * address cannot be looked up.
 */
tc_status_t tc_forward_noalloc(const tc_shape_t* shape, const void* q, const void* k, const void* v,
                               const float* lambda, const float* eta, const float* gate, void* y,
                               float* A_final, float* lse, void* stream);

/*
 * tc_decode_step -- one streaming step (Figure 2, steps 1-5) for S streams.
 *   q, k, v  [S,H,D] dtype: the incoming token of every (stream, head).
 *   k_ring, v_ring [S,H,W,D] dtype, in/out: token t lives in slot t mod W.
 *   A        [S,H,D,D] float32, in/out: the eviction memory.
 *   pos      [S] int64, in/out: index of the incoming token of each stream;
 *            incremented by one.
 * With t = pos[s], slot = t mod W, per head: if t >= W the pair in the slot
 * is evicted and written, A <- lambda*A + eta*k_e v_e^T; the new pair takes
 * the slot; y = softmax over the min(t+1, W) resident pairs + sigmoid(g)*q A.
 *   y        [S,H,D] dtype, out.
 * Rings, A and pos are updated in place, so successive calls need no host
 * work between them (the sequence can be captured in a HIP graph).
 * One (stream, head) ring must stay below 2 GiB ((W + 512) * D * element
 * size < 2^31), else TC_ERR_UNSUPPORTED.
 */
tc_status_t tc_decode_step(const tc_decode_shape_t* shape, const void* q, const void* k,
                           const void* v, void* k_ring, void* v_ring, float* A, int64_t* pos,
                           const float* lambda, const float* eta, const float* gate, void* y,
                           void* stream);

/*
 * tc_forward_continue -- chunked prefill after earlier tokens, and the
 * prefill -> decode handoff (Figure 2: a stream's layer state is the ring of
 * its last W pairs and the memory A; Section 3.2 write-on-evict).  The batch
 * has seen pos0 tokens per sequence (a host value, the same for all B);
 * this call takes the next T tokens, positions pos0 .. pos0+T-1, and gives
 * exactly what T successive tc_decode_step calls give (up to float
 * rounding), computed with the parallel forward.  With pos0 = 0 the outputs
 * equal tc_forward's, and the ring/A it leaves are the state a decode at
 * position T continues from.
 *   shape    B, H, T (new tokens), D, W, C, scale, dtype as for tc_forward.
 *   q, k, v  [B,H,T,D] dtype: the new tokens.
 *   k_ring, v_ring [B,H,W,D] dtype, in/out: token t in slot t mod W (the
 *            tc_decode_step layout with S = B).  On entry the slots of the
 *            last min(pos0, W) tokens are read; on return they hold the last
 *            min(pos0 + T, W) tokens (other slots are left as they are).
 *   A        [B,H,D,D] float32, in/out: the memory after step pos0-1 on
 *            entry (zero for pos0 <= W: nothing was evicted), after step
 *            pos0+T-1 on return.
 *   pos      [B] int64, out, nullable: set to pos0 + T (the decode position).
 *   y        [B,H,T,D] dtype, out.   lse [B,H,T] float32, out, nullable.
 *   ws       device workspace of at least tc_continue_workspace_size(shape,
 *            pos0) bytes: the forward's segment states and flags for the
 *            extended sequence of min(pos0, W) + T rows (the ring prefix, then
 *            the new tokens, both read in place: nothing is copied), and
 *            float32 room for the read of A when the forward cannot start its
 *            scan from A (pos0 < W, or W not a multiple of the forward's
 *            block rows: 128 for bf16 with D <= 64, else 64).
 * Every pointer must be 16-byte aligned.  Outputs (rings, A, pos, y, lse,
 * ws) must not overlap the inputs or each other.  The extended sequence is
 * subject to the tc_forward size limits (TC_ERR_UNSUPPORTED otherwise).
 */
size_t tc_continue_workspace_size(const tc_shape_t* shape, int64_t pos0);
tc_status_t tc_forward_continue(const tc_shape_t* shape, int64_t pos0, const void* q, const void* k,
                                const void* v, const float* lambda, const float* eta,
                                const float* gate, void* k_ring, void* v_ring, float* A,
                                int64_t* pos, void* y, float* lse, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * tc_forward_status -- whether every flag wait of the last forward call that
 * used workspace `ws` completed (the state exchange of tc_forward, Section
 * 3.2: each row must read the true state of all evictions before it).
 *   shape, pos0   the call's shape; pos0 = 0 for tc_forward, the call's pos0
 *                 for tc_forward_continue (its workspace holds a forward
 *                 workspace of the extended sequence at offset 0).
 *   ws, ws_bytes  that call's workspace.
 * Synchronises `stream` (the call's stream), copies the per-workgroup status
 * words to the host and returns TC_OK, or TC_ERR_STATE_EXCHANGE when a wait
 * ran out (the call's NaN rows).  TC_OK as well when the shape needs no
 * workspace (one segment per sequence: nothing to wait for).  Validation
 * errors as for the call itself; TC_ERR_HIP if the synchronisation or the
 * copy fails.  Calls that wrote the same workspace later overwrite the words.
 */
tc_status_t tc_forward_status(const tc_shape_t* shape, int64_t pos0, const void* ws, size_t ws_bytes,
                              void* stream);

/*
 * tc_backward -- gradients of L = sum_t <dy_t, y_t> through both levels and
 * the scan (the abstract: decay, write rate and gate are trained end to end).
 *   q, k, v, y, dy [B,H,T,D] dtype: forward inputs, forward output, upstream
 *            gradient.
 *   lse      [B,H,T] float32: from tc_forward.
 *   dq, dk, dv [B,H,T,D] dtype, out.
 *   dlambda, deta, dgate [H] float32, out (overwritten): summed over B and T.
 *   ws       device workspace of at least tc_backward_workspace_size bytes.
 */
tc_status_t tc_backward(const tc_shape_t* shape, const void* q, const void* k, const void* v,
                        const void* y, const void* dy, const float* lse, const float* lambda,
                        const float* eta, const float* gate, void* dq, void* dk, void* dv,
                        float* dlambda, float* deta, float* dgate, void* ws, size_t ws_bytes,
                        void* stream);

/* Static description of a status code. */
const char* tc_status_string(tc_status_t status);

/* Library version, e.g. "0.1.0". */
const char* tc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TC_H_ */
