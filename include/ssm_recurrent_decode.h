/*
 * ssm_recurrent_decode.h -- C ABI of the MI355X (gfx950) batched single-token SSM
 * decode library (libssm_recurrent_decode.so).
 *
 * What is computed comes from "ReplaySSM: Cache SSM Inputs, Not State" (a summary
 * of Tri Dao's blog post); each entry point names the section it follows.  The
 * conv state layout comes from the vLLM page on disaggregated prefill/decode for
 * hybrid SSM models, section "DS Layout".
 *
 * General rules
 * -------------
 *  - Every pointer argument is a DEVICE pointer (hipMalloc'd or equivalent) owned
 *    by the caller, unless stated otherwise.  The library never allocates, frees,
 *    copies to the host or synchronises; a call validates its arguments on the
 *    host, enqueues its kernels on `stream` and returns.  Every call is therefore
 *    safe to capture in a HIP graph (no memset nodes are recorded).
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 *  - Return value: 0 = enqueued.  Negative = rejected on the host before anything
 *    was enqueued: RSSM_EINVAL (null pointer, non-positive or inconsistent size,
 *    H % G != 0, T < 1, L < 2T for a verify), RSSM_ENOTSUP (a (d, n, L, T) the
 *    library was not built for), RSSM_ELAUNCH (the HIP launch itself failed).
 *  - Device-side anomalies in the ring pointers (head/count/pending out of range,
 *    accepted > pending, drafts left uncommitted) never fault: the kernels clamp
 *    the value into range, proceed, and OR a bit into *ring->err (when err is not
 *    NULL).  The caller reads that word whenever it chooses.
 *  - Dense row-major layouts, innermost index last.  bf16 is passed as its
 *    uint16_t bit pattern.  fp32 is IEEE binary32.
 *  - Every array is 16-byte aligned (the kernels move 16-byte chunks; hipMalloc
 *    returns 256-byte aligned memory), rssm_ring.meta 128-byte aligned and
 *    rssm_ring.err 4-byte aligned; a misaligned pointer is RSSM_EINVAL.
 *  - Outputs must not alias inputs.  Different requests are independent, so two
 *    calls on disjoint buffers may run on different streams concurrently; two
 *    calls on the same ring must be ordered (same stream or events).
 *
 * Symbols: B batch, H nheads, d head_dim, n state_dim, G ngroups (head h reads
 * the k/q of group h / (H / G)), L ring capacity, T draft window.
 * Supported: d in {64, 128}; n in {64, 128, 256} for every call, RSSM_ENOTSUP
 * otherwise; 1 <= L <= 32; 1 <= T <= 8 with 2T <= L for
 * the verify calls; any B >= 1, H >= 1 with H % G == 0 and B * H < 2^24 (one
 * 256-thread work-group per (request, head); larger: RSSM_EINVAL).
 */
#ifndef SSM_RECURRENT_DECODE_H
#define SSM_RECURRENT_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSSM_ABI_VERSION 11

#define RSSM_OK 0
#define RSSM_EINVAL (-22)
#define RSSM_ENOTSUP (-95)
#define RSSM_ELAUNCH (-5)

/* bits OR-ed into *ring->err by the kernels */
#define RSSM_ERR_POINTERS 1  /* head/count/pending out of range on entry (clamped)       */
#define RSSM_ERR_ACCEPTED 2  /* accepted[b] outside [0, pending[b]] (clamped)            */
#define RSSM_ERR_PENDING 4   /* decode/verify called with uncommitted drafts (dropped)   */
#define RSSM_ERR_SLOT 8      /* slots[b] >= rows: batch entry b skipped                   */
#define RSSM_ERR_DIVERGED 16 /* the H records of one request hold different pointer words  */

typedef struct rssm_dims {
  int32_t batch;      /* B */
  int32_t nheads;     /* H */
  int32_t head_dim;   /* d: value / output length, rows of the per-head state */
  int32_t state_dim;  /* n: key / query length, columns of the per-head state  */
  int32_t ngroups;    /* G: k and q are shared by the H/G heads of a group     */
  int32_t capacity;   /* L: ring capacity (ignored by the standard-step calls) */
  int32_t flags;      /* RSSM_F_* storage-precision options; 0 = fp32 y and GDN u   */
} rssm_dims;

/*
 * Storage-precision options (the precision the method page's serving setup keeps
 * decode vectors in: bf16; the default here is fp32 for y and for the GDN
 * corrections, see each entry point).  Unknown bits: RSSM_EINVAL.
 *   RSSM_F_Y_BF16  outputs y stored as bf16 (round to nearest even) instead of
 *                  fp32, same shape; honoured by replay_append_decode(_conv),
 *                  replay_verify_T, gdn_replay_verify_T, gdn_replay_append_decode;
 *                  the standard-step and snapshot calls return RSSM_ENOTSUP.
 *   RSSM_F_U_BF16  GDN rings cache the corrections u as bf16 [B, H, L, d] (a
 *                  property of the ring: every call on it must carry the flag, and
 *                  rssm_ring_sizes sizes vu by it).  The outputs of the call that
 *                  computes u use it unrounded; later calls (and a fold) read the
 *                  rounded value.  Mamba-2 calls ignore it.
 */
#define RSSM_F_Y_BF16 1
#define RSSM_F_U_BF16 2

/*
 * Per-request ReplaySSM decode memory besides the checkpoint state S_0.
 * (Method, "core idea" and "three advantages"; kernel design, "ring buffer".)
 * The ring holds the most recent inputs since the checkpoint, addressed modulo L
 * from `head`, so a rollback only moves a pointer.  Physical slot of logical
 * entry j (0 = oldest) of request b is (head + j) % L.
 *
 * Values (Mamba-2 v) and corrections (GDN u) are stored in blocks of hb
 * consecutive heads, vu[B][H / hb][L][hb][d] with hb = RSSM_RING_HEAD_BLOCK(H)
 * (4 when H % 4 == 0, else 2 when H is even, else 1): entry `slot` of head h of
 * request b starts at element (((b * (H / hb) + h / hb) * L + slot) * hb + h % hb) * d.
 * The entries a call caches for the heads of a block are adjacent in memory.
 *
 * Everything else a call needs about request b's ring as head h sees it sits in
 * one record (rssm_ring_record below) of RSSM_META_WORDS(L) 32-bit words: one
 * 128-byte line for L <= 29, two for larger L.  The records of a ring are
 * meta[(b * H + h) * RSSM_RECORD_LINES(L) + ...], and each holds
 *   ptr         the pointer word (RSSM_PTR_* below): head, count = committed
 *               entries since the checkpoint, pending = uncommitted drafts that
 *               follow them;
 *   A           Mamba-2: the head's A of the cached entries (so a flush needs no
 *               parameters); GDN: unused;
 *   slot s      (RSSM_RECORD_SLOT(rec, s), s < L; for L > 29 the slots run on
 *               into the record's second line) Mamba-2: Delta after softplus
 *               (the decay is a = exp(A Delta)); GDN: alpha = exp(g).
 * A call writes each record it moves as whole lines, so the per-step bookkeeping
 * costs one full-line write per head instead of several partial ones.  Every
 * call moves all H records of a request the same way, so their pointer words
 * stay equal; the work of head h reads and writes only record h, so no two
 * work-groups share one and no atomics are needed.  rssm_ring_pointers gives
 * the per-request int32 view of the pointer words on the device.
 *
 * Caller allocates every array (meta 128-byte aligned) and zero-fills meta and
 * err once before the first call; afterwards only the library writes them
 * (rssm_ring_reset re-zeroes the pointer words of a subset of requests).
 * Unsigned fields: a head >= L or a count above the largest legal value is
 * clamped and flagged (RSSM_ERR_POINTERS).  Bits 48-63 of the word are zero.
 *
 * Pooled rings (serving layout).  With slots == NULL, batch entry b owns row b
 * of state0 and of the ring arrays.  With slots != NULL, state0, vu, k and meta
 * hold `rows` request rows -- a block pool in which one block is one request's
 * whole decode state -- and batch entry b of a call works on row slots[b]; the
 * call's own inputs and outputs (v, k, q, dt, g, beta, y, flushed, accepted,
 * mask) stay indexed by b.  A negative slot marks a padding entry (a batch
 * padded up to a captured size): it is skipped, nothing of it read or written.
 * slots[b] >= rows: skipped, RSSM_ERR_SLOT flagged.  Two entries of one call
 * must not name the same row.  Sizes: rssm_ring_sizes with dims->batch = rows.
 */
#define RSSM_RING_HEAD_BLOCK(H) ((H) % 4 == 0 ? 4 : ((H) % 2 == 0 ? 2 : 1))
#define RSSM_META_WORDS(L) ((L) + 3 <= 32 ? 32 : 64)
#define RSSM_RECORD_LINES(L) (RSSM_META_WORDS(L) / 32)
#define RSSM_PTR_HEAD(w) ((uint32_t)((w) & 0xFFFFu))
#define RSSM_PTR_COUNT(w) ((uint32_t)(((w) >> 16) & 0xFFFFu))
#define RSSM_PTR_PENDING(w) ((uint32_t)(((w) >> 32) & 0xFFFFu))
#define RSSM_PTR_PACK(head, count, pending)                                \
  (((uint64_t)(head) & 0xFFFFu) | (((uint64_t)(count) & 0xFFFFu) << 16) | \
   (((uint64_t)(pending) & 0xFFFFu) << 32))

/* One 128-byte line of a ring record (see above). */
typedef struct rssm_ring_record {
  uint64_t ptr;     /* pointer word (RSSM_PTR_*)                                  */
  float A;          /* Mamba-2: A of the cached entries; GDN: unused              */
  float slot[29];   /* per physical slot: Delta (Mamba-2) or alpha (GDN); slots
                       29..L-1 of a two-line record continue in the next line    */
} rssm_ring_record;
/* Slot s of the record starting at rec (any s < L, either line). */
#define RSSM_RECORD_SLOT(rec, s) (((float*)(rec))[3 + (s)])

typedef struct rssm_ring {
  void* vu;          /* Mamba-2: v bf16, GDN: u fp32 (or bf16, RSSM_F_U_BF16),
                        [B, H / hb, L, hb, d] (see above)                            */
  uint16_t* k;       /* bf16 [B, G, L, n]                                           */
  rssm_ring_record* meta;  /* [B, H, RSSM_RECORD_LINES(L)] records (see above)     */
  int32_t* err;      /* [1] anomaly bits (RSSM_ERR_*), may be NULL                  */
  const int32_t* slots;  /* [B] pool row of each batch entry, or NULL (row = b)     */
  int32_t rows;      /* pool rows when slots != NULL (>= 1); ignored otherwise       */
} rssm_ring;

int rssm_abi_version(void);
const char* rssm_strerror(int code);

/* Bytes of each ring array for the given dims: writes 4 sizes in the order of
 * the rssm_ring fields (vu, k, meta, err).  is_gdn selects fp32 u instead of
 * bf16 v.  Host-only. */
int rssm_ring_sizes(const rssm_dims* dims, int is_gdn, size_t out_bytes[4]);

/* Zero the pointer words (head, count, pending) of requests with
 * mask[b] != 0 (mask NULL = all) and clear err.  The ring contents are left as
 * they are: with count = 0 they are never read.  Use after an explicit
 * replay_flush to recycle a request slot, or to start a new request from a
 * checkpoint state. */
int rssm_ring_reset(const rssm_dims* dims, rssm_ring* ring, const int32_t* mask, void* stream);

/*
 * The ring pointers of every request as int32 arrays, written on the device
 * (CUDA-Graph notes, "device-side commit and rollback": the pointers live on the
 * GPU and are moved there by kernels, so a scheduler that needs them -- to size
 * the next window, to spot requests about to flush -- reads them without a host
 * synchronisation, and the call can sit inside a captured graph).
 *   head[b], count[b], pending[b]  int32 [B] out, each may be NULL: the fields
 *        of request b's pointer word (its row slots[b] in a pooled ring;
 *        padding entries and rows outside the pool get -1 in every field)
 * The call also compares the H records of each request and ORs
 * RSSM_ERR_DIVERGED into *ring->err when their pointer words differ (only
 * possible after a write outside the library); the fields then come from head
 * 0's record.  Works on Mamba-2 and GDN rings alike; the ring is only read.
 */
int rssm_ring_pointers(const rssm_dims* dims, const rssm_ring* ring, int32_t* head, int32_t* count,
                       int32_t* pending, void* stream);

/* ---------------------------------------------------------------- Mamba-2 */

/*
 * Standard Mamba-2 decode step with state write-back (the baseline).
 * Background, "memory-bound": S_t = a_t S_{t-1} + Delta_t v_t k_t^T, y_t = S_t q_t,
 * a_t = exp(A Delta_t); algorithms, "Mamba-2 standard decode", baseline bullet.
 *   state   fp32 [B, H, d, n]  in/out
 *   v       bf16 [B, H, d];  k, q bf16 [B, G, n]
 *   dt      fp32 [B, H] raw step; Delta = softplus(dt + dt_bias[h])
 *   dt_bias fp32 [H];  A fp32 [H] (negative)
 *   y       fp32 [B, H, d]  out
 */
int ssm_decode_step(const rssm_dims* dims, float* state, const uint16_t* v, const uint16_t* k,
                    const uint16_t* q, const float* dt, const float* dt_bias, const float* A,
                    float* y, void* stream);

/*
 * ReplaySSM append-decode for one token per request.
 * Algorithms, "Mamba-2 standard decode", ReplaySSM bullet; method, "output-only
 * decode": append (v, Delta, k) to the ring (the decay a = exp(A Delta) is
 * recomputed from Delta and the A kept in the record); with the c entries
 * since the checkpoint (this one included),
 *     y = abar (S_0 q) + sum_j s_j (k_j^T q) v_j,
 *     abar = prod_i a_i,  s_j = Delta_j prod_{i>j} a_i;
 * S_0 is only read.  When the append fills the ring (c == L) the same call
 * flushes: S_0 <- abar S_0 + sum_j s_j v_j k_j^T, head advances by L, count = 0.
 * The flush decision is per request, read from count at run time.
 *   state0  fp32 [B, H, d, n] checkpoint, read (written on flush steps)
 *   ring    Mamba-2 ring; requires pending == 0 and count < L on entry
 *   v, k, q, dt, dt_bias, A, y  as ssm_decode_step; A must be the same in every
 *           call while entries are cached (the cached decays are exp(A Delta))
 *   flushed int32 [B] out (1 = this request flushed), may be NULL
 */
int replay_append_decode(const rssm_dims* dims, float* state0, rssm_ring* ring,
                         const uint16_t* v, const uint16_t* k, const uint16_t* q,
                         const float* dt, const float* dt_bias, const float* A, float* y,
                         int32_t* flushed, void* stream);

/*
 * replay_append_decode with the layer's front-end fused in: the token's v, k, q
 * are produced in the same launch by the causal depthwise conv1d (width 4) with
 * SiLU over the layer's xBC channels, the step before the mixer (vLLM hybrid
 * page: conv state (dim, state_len), "DS" layout), instead of being read as
 * inputs.  Channel order of xBC (C = H d + 2 G n channels): x of head h at
 * h d .. h d + d - 1 (-> v), B of group g at H d + g n .. (-> k), C of group g at
 * H d + G n + g n .. (-> q).  Per channel, window = [state[0..2], xbc]:
 *     out = SiLU(sum_w conv_w[c, w] window[w]),  new state = window[1..3];
 * v, k, q = out rounded to bf16 (nearest even), then the ReplaySSM step exactly
 * as replay_append_decode.
 *   conv_state_in  bf16 [B, C, 3] (pooled: [rows, C, 3]) read
 *   conv_state_out bf16 [B, C, 3] written; must not be conv_state_in (the heads
 *                  of a group read B and C states while they write them):
 *                  swap the two buffers every step
 *   xbc bf16 [B, C];  conv_w bf16 [C, 4] (no bias);  other arguments as
 *   replay_append_decode.
 */
int replay_append_decode_conv(const rssm_dims* dims, float* state0, rssm_ring* ring,
                              const uint16_t* conv_state_in, uint16_t* conv_state_out,
                              const uint16_t* xbc, const uint16_t* conv_w, const float* dt,
                              const float* dt_bias, const float* A, float* y, int32_t* flushed,
                              void* stream);

/*
 * Explicit flush of the committed entries (method, "core idea": summarise the
 * buffered inputs into the state and clear the buffer).  For requests with
 * mask[b] != 0 (mask NULL = all) and count > 0:
 *     S_0 <- abar S_0 + sum_{j<count} s_j v_j k_j^T ;  head += count ;  count = 0.
 * Pending drafts stay cached after the new head.  The decays come from the Delta
 * and A kept in each record by the calls that cached the entries.
 */
int replay_flush(const rssm_dims* dims, float* state0, rssm_ring* ring, const int32_t* mask,
                 void* stream);

/*
 * ReplaySSM speculative verify of T drafts per request.
 * Algorithms, "speculative decoding", ReplaySSM bullet and the flush-decision
 * rule: drafts go to the slots after the c committed entries; draft s (0-based)
 * sees p_s = c + s + 1 entries:
 *     y_s = abar_s (S_0 q_s) + sum_{j<p_s} w_{j,s} (k_j^T q_s) v_j,
 *     abar_s = prod_{i<p_s} a_i,  w_{j,s} = Delta_j prod_{j<i<p_s} a_i.
 * If c + 2T > L the c committed entries (never the drafts) are folded into S_0
 * in the same call (head += c, count = 0), so at least T slots stay free for the
 * next window.  pending becomes T; replay_rollback commits the accepted prefix.
 *   v bf16 [B, T, H, d];  k, q bf16 [B, T, G, n];  dt fp32 [B, T, H] raw
 *   y fp32 [B, T, H, d] out (every draft position, rejected ones included)
 *   flushed int32 [B] out, may be NULL
 *   dt_bias, A as replay_append_decode (A the same while entries are cached)
 * Requires 1 <= T, 2T <= L; on entry pending == 0 and count + T <= L.
 */
int replay_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                    const uint16_t* v, const uint16_t* k, const uint16_t* q, const float* dt,
                    const float* dt_bias, const float* A, float* y, int32_t* flushed,
                    void* stream);

/*
 * Device-side commit / rollback (method, "rollback becomes a buffer operation";
 * CUDA-Graph notes, "device-side commit and rollback"): for every request
 *     count += clamp(accepted[b], 0, pending[b]);  pending = 0.
 * Rejected drafts are simply left beyond count.  No host synchronisation.
 * Shared by the Mamba-2 and GDN rings (it touches pointers only).
 *   accepted int32 [B] (device)
 */
int replay_rollback(const rssm_dims* dims, rssm_ring* ring, const int32_t* accepted,
                    void* stream);

/*
 * replay_verify_T with the commit of the previous window folded in: for every
 * request that holds pending drafts (left by the previous verify on this ring),
 *     count += clamp(accepted[b], 0, pending);  pending = 0,
 * exactly as replay_rollback would, then the verify of the T new drafts as
 * replay_verify_T (the early-flush decision taken from the committed count).
 * One launch per speculative round instead of two (CUDA-Graph notes,
 * "device-side commit and rollback": the commit stays on the device; here it
 * also shares the verify's launch).  Requests with no pending drafts ignore
 * accepted[b].  The last window of a run is committed with replay_rollback.
 *   accepted int32 [B] (device): the previous window's accepted drafts of the
 *            request at batch entry b of this call (with a slot map: of row
 *            slots[b], wherever that request sat in the previous call)
 *   other arguments as replay_verify_T
 */
int replay_commit_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                           const int32_t* accepted, const uint16_t* v, const uint16_t* k,
                           const uint16_t* q, const float* dt, const float* dt_bias, const float* A,
                           float* y, int32_t* flushed, void* stream);

/* ---------------------------------------------------------- Gated DeltaNet */

/*
 * Standard GDN decode step with state write-back (baseline).
 * Background: S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 * y_t = S_t q_t; computed as u = beta (v - e^g S k), S <- e^g S + u k^T.
 *   state fp32 [B, H, d, n] in/out;  v bf16 [B, H, d];  k, q bf16 [B, G, n]
 *   g, beta fp32 [B, H] (already activated: g <= 0, 0 < beta < 1)
 *   y fp32 [B, H, d] out
 */
int gdn_decode_step(const rssm_dims* dims, float* state, const uint16_t* v, const uint16_t* k,
                    const uint16_t* q, const float* g, const float* beta, float* y,
                    void* stream);

/*
 * ReplaySSM GDN speculative verify (appendix, "GDN speculative decoding" and
 * "GDN standard decode").  The ring caches the corrections u (fp32) with k and
 * alpha = e^g.  With the committed state S_h = abar S_0 + sum_j w_j u_j k_j^T
 * read only through products with the 2T draft vectors, gamma_s = prod_{i<=s}
 * alpha_i over the window:
 *     R_s = beta_s (v_s - gamma_s S_h k_s),
 *     A_{s,s'} = beta_s (gamma_s / gamma_s') (k_s . k_s')   (s' < s),
 *     (I + A) U = R  (strictly lower-triangular T x T solve),
 *     y_s = gamma_s S_h q_s + sum_{s'<=s} (gamma_s / gamma_s') (k_s' . q_s) u_s'.
 * (u_s, k_s, alpha_s) are written after the committed entries; early flush of
 * the committed entries when c + 2T > L, as replay_verify_T; pending = T.
 *   v bf16 [B, T, H, d];  k, q bf16 [B, T, G, n];  g, beta fp32 [B, T, H]
 *   y fp32 [B, T, H, d] out;  flushed int32 [B] out, may be NULL
 */
int gdn_replay_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                        const uint16_t* v, const uint16_t* k, const uint16_t* q, const float* g,
                        const float* beta, float* y, int32_t* flushed, void* stream);

/* gdn_replay_verify_T with the previous window's commit folded in, as
 * replay_commit_verify_T. */
int gdn_replay_commit_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                               const int32_t* accepted, const uint16_t* v, const uint16_t* k,
                               const uint16_t* q, const float* g, const float* beta, float* y,
                               int32_t* flushed, void* stream);

/*
 * ReplaySSM GDN standard decode, one token per request (appendix, "GDN standard
 * decode"; method, "core idea": flush when the ring is full).  With the c
 * entries since the checkpoint, S_c = abar S_0 + sum_j w_j u_j k_j^T read only
 * through S_c k and S_c q:
 *     u = beta (v - alpha S_c k),  y = alpha S_c q + (k . q) u,  alpha = e^g;
 * (u, k, alpha) is cached as entry c and committed in the same call (count + 1).
 * When this append fills the ring (c + 1 == L) the same call folds all L entries:
 * S_0 <- prod alpha S_0 + sum_j w_j u_j k_j^T, count = 0.
 *   state0 fp32 [B, H, d, n];  ring GDN ring, pending == 0 and count < L on entry
 *   v bf16 [B, H, d];  k, q bf16 [B, G, n];  g, beta fp32 [B, H] (as gdn_decode_step)
 *   y fp32 [B, H, d] out;  flushed int32 [B] out, may be NULL
 */
int gdn_replay_append_decode(const rssm_dims* dims, float* state0, rssm_ring* ring,
                             const uint16_t* v, const uint16_t* k, const uint16_t* q,
                             const float* g, const float* beta, float* y, int32_t* flushed,
                             void* stream);

/*
 * Explicit GDN flush (appendix, state-and-output route): for requests with
 * mask[b] != 0 (NULL = all) and count > 0,
 *     S_0 <- abar S_0 + sum_{j<count} w_j u_j k_j^T,  w_j = prod_{j<i<count} alpha_i,
 * head += count, count = 0.
 */
int gdn_replay_flush(const rssm_dims* dims, float* state0, rssm_ring* ring, const int32_t* mask,
                     void* stream);

/* ---------------------------------------------------------- speculative baseline */

/*
 * The speculative-decoding route that ReplaySSM replaces (background, "the cost
 * of summarising": one full state snapshot kept per draft and restored on
 * rejection; algorithms, "speculative decoding", baseline bullet: serial state
 * update per draft position).  Every request owns nslots = P >= T + 1 state
 * slots and slot[b] names the committed one.  The T drafts run serially from it
 * and the state after draft s is stored, whole, into slot (slot[b] + 1 + s) mod P;
 *     y_s = S_s q_s,  S_s the state after drafts 0..s.
 * Restoring the snapshot of the last accepted draft is snapshot_commit's move of
 * slot[b].  Per head and round: 4dn bytes read, T * 4dn bytes written.
 *   pool  fp32 [B, P, H, d, n]: slot[b] read, the T slots after it overwritten
 *   slot  int32 [B] (device), read only here; outside [0, P) it is reduced mod P
 *         and RSSM_ERR_POINTERS is OR-ed into *err (err may be NULL)
 *   Mamba-2: v bf16 [B, T, H, d]; k, q bf16 [B, T, G, n]; dt fp32 [B, T, H] raw;
 *            dt_bias, A fp32 [H] (as ssm_decode_step)
 *   GDN:     v, k, q as above; g, beta fp32 [B, T, H] (as gdn_decode_step)
 *   y fp32 [B, T, H, d] out
 * dims->capacity is not used.  Requires 1 <= T <= 8 and nslots >= T + 1.
 */
int ssm_snapshot_verify_T(const rssm_dims* dims, int32_t T, int32_t nslots, float* pool,
                          const int32_t* slot, const uint16_t* v, const uint16_t* k,
                          const uint16_t* q, const float* dt, const float* dt_bias, const float* A,
                          float* y, int32_t* err, void* stream);
int gdn_snapshot_verify_T(const rssm_dims* dims, int32_t T, int32_t nslots, float* pool,
                          const int32_t* slot, const uint16_t* v, const uint16_t* k,
                          const uint16_t* q, const float* g, const float* beta, float* y,
                          int32_t* err, void* stream);

/*
 * Commit of the snapshot route, on the device: for every request
 *     slot[b] <- (slot[b] + clamp(accepted[b], 0, T)) mod nslots,
 * so the snapshot after the last accepted draft becomes the committed state
 * (accepted 0 keeps the old one).  Out-of-range accepted or slot values are
 * clamped / reduced and flagged (RSSM_ERR_ACCEPTED, RSSM_ERR_POINTERS) in *err.
 *   slot int32 [B] in/out;  accepted int32 [B];  err int32 [1], may be NULL
 */
int snapshot_commit(int32_t batch, int32_t T, int32_t nslots, int32_t* slot,
                    const int32_t* accepted, int32_t* err, void* stream);

/* ---------------------------------------------------------- causal conv1d */

/*
 * Fused causal depthwise conv1d state update with SiLU, one token per request.
 * The conv state is stored channel-major with the time axis fastest, the
 * (dim, state_len) "DS" layout of the vLLM disaggregation page.  With
 * window = [state[b,c,0..W-2], x[b,c]]:
 *     out[b,c] = SiLU(sum_w weight[c,w] window[w]);  state[b,c,:] <- window[1..W-1].
 *   conv_state bf16 [B, C, W-1] in/out;  x bf16 [B, C];  weight bf16 [C, W]
 *   out fp32 [B, C]
 * Supported: W = 4 and an even number of channels C; otherwise RSSM_ENOTSUP.
 */
int causal_conv1d_update(int32_t batch, int32_t channels, int32_t width, uint16_t* conv_state,
                         const uint16_t* x, const uint16_t* weight, float* out, void* stream);

/* ---------------------------------------------------------- measurement aid */

/*
 * Streaming HBM probes used to calibrate traffic counters and to record the
 * achievable bandwidth: rssm_probe_copy copies `bytes` (multiple of 16) from
 * src to dst; rssm_probe_read reads `bytes` and writes one fp32 checksum per
 * work-group into sink (sink holds at least rssm_probe_read_sink_floats(bytes)).
 */
int rssm_probe_copy(void* dst, const void* src, size_t bytes, void* stream);
int rssm_probe_read(const void* src, size_t bytes, float* sink, void* stream);
size_t rssm_probe_read_sink_floats(size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* SSM_RECURRENT_DECODE_H */
