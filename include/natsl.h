/*
 * natsl.h -- C ABI of the NAtS-L hybrid attention layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (gist.science, "Technische Samenvatting: Neural Attention Search
 * Linear (NAtS-L)", section Kernmechanismen, items 1-4; the German
 * "Technisches Resümee" of the same paper repeats it):
 *   1. the sequence is split into chunks of 64 tokens ("Die Chunking-
 *      Strategie" in the German explainer); an Attention Score Layer (mean-
 *      pool of the chunk, then a linear layer) scores each chunk for the two
 *      operation types and the highest score picks the chunk's operation:
 *      softmax attention or Gated DeltaNet;
 *   3. both operations are computed inside every chunk; at the chunk's end
 *      only the selected operation keeps the chunk (softmax keeps its KV,
 *      Gated DeltaNet keeps its state update; the other rolls back to the
 *      chunk start);
 *   4. both outputs are RMS-normalised and mixed with weights derived from Q.
 *
 * Conventions shared by every entry point:
 *   - every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or synchronises device memory;
 *   - scratch memory is a caller-provided workspace whose size comes from
 *     natsl_workspace_size(); it must be 256-byte aligned;
 *   - every call is asynchronous on the caller's stream (natsl_forward,
 *     natsl_nha_attention and natsl_gdn_backward with the overlap workspace
 *     fork work onto a library-owned helper stream of default priority and
 *     join it back before returning, also when they fail after the fork; the
 *     join is an event wait, not a host synchronisation);
 *   - threads: every entry point may be called from several host threads at
 *     once, on the same or different streams.  The library keeps no mutable
 *     state between calls except (a) helper streams and their events, which
 *     those calls take from a per-device pool for the duration of their
 *     enqueue, so concurrent calls never share them, (b) a record of the
 *     kernels whose LDS limit has been raised, guarded by a mutex, and (c)
 *     the natsl_profile_* timing records, guarded by a mutex (timing several
 *     threads at once mixes their records), (d) the scratch array of
 *     natsl_decode_step_noalloc (see there), and (e) the level of the
 *     natsl_set_sync_check debug mode (atomic).  Calls whose device buffers
 *     overlap must be ordered by the caller (same stream, or events);
 *   - every call validates its arguments on the host BEFORE enqueueing any
 *     work; on failure nothing is enqueued, a status != NATSL_OK is
 *     returned and natsl_last_error() (thread-local) describes the problem;
 *   - a failed HIP launch returns NATSL_ERR_DEVICE;
 *   - results are bit-identical from run to run (no float atomics);
 *   - tensors are dense row-major with the shapes given; io tensors (x, q, k,
 *     v, out) hold the io dtype of natsl_dims, alpha/beta/weights are fp32;
 *   - supported: Dk == Dv in {64, 128}, chunk == 64, L % 64 == 0, L >= 64,
 *     B * H * L <= 2^28 (so that every launch's work-item count stays
 *     below 2^32; q, k, v and out alone take 256 GiB at that bound),
 *     route_groups G in {1, H}, H <= 1024, d_model % 8 == 0
 *     and 8 <= d_model <= 32768 (where d_model is used).  The Gated DeltaNet
 *     branch (natsl_gdn_chunk, natsl_forward) with bf16 io and D = 128 takes
 *     at most 15232 chunks per sequence (L <= 974848); a longer L is
 *     NATSL_ERR_UNSUPPORTED before anything is enqueued.  B == 0 is a no-op
 *     that succeeds after the dims check (tensor pointers may then be NULL).
 *   - route ids: 0 = softmax attention, 1 = Gated DeltaNet (linear).
 */
#ifndef NATSL_H
#define NATSL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NATSL_OK = 0,
  NATSL_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent dims */
  NATSL_ERR_UNSUPPORTED = 2,  /* valid but outside what v1 implements      */
  NATSL_ERR_WORKSPACE = 3,    /* workspace missing, misaligned or too small */
  NATSL_ERR_DEVICE = 4,       /* a HIP call or kernel launch failed         */
  NATSL_ERR_CAPACITY = 5      /* host-visible capacity problem (decode)     */
} natsl_status;

typedef enum {
  NATSL_F32 = 0,
  NATSL_BF16 = 1,
  /* Not dtypes: these two make natsl_dtype a full 32-bit signed integer in C
   * and in C++, so that any int a caller stores in a dtype field is a value of
   * the type (the library then rejects it with NATSL_ERR_INVALID_ARG) rather
   * than undefined behaviour in the library's C++. */
  NATSL_DTYPE_MIN_ = -2147483647 - 1,
  NATSL_DTYPE_MAX_ = 2147483647
} natsl_dtype;

enum { NATSL_ROUTE_SOFTMAX = 0, NATSL_ROUTE_LINEAR = 1 };

/* entry ids for natsl_workspace_size */
enum {
  NATSL_ENTRY_ROUTE = 0,
  NATSL_ENTRY_GDN_CHUNK = 1,
  NATSL_ENTRY_SOFTMAX_MASKED = 2,
  NATSL_ENTRY_MERGE = 3,
  NATSL_ENTRY_FORWARD = 4,
  NATSL_ENTRY_DECODE_STEP = 5,
  NATSL_ENTRY_DECODE_HANDOFF = 6,
  NATSL_ENTRY_SOFTMAX_BACKWARD = 7,
  NATSL_ENTRY_GDN_BACKWARD = 8,
  NATSL_ENTRY_MERGE_BACKWARD = 9,
  NATSL_ENTRY_ROUTE_BACKWARD = 10,
  NATSL_ENTRY_GDN_BACKWARD_OVERLAP = 11  /* natsl_gdn_backward's larger, overlapping layout */
};

typedef struct {
  int32_t B, H, L;        /* batch, heads, sequence length (decode: L unused) */
  int32_t Dk, Dv;         /* head dims (Dk == Dv in v1)                        */
  int32_t d_model;        /* width of the router input x                       */
  int32_t chunk;          /* must be 64                                        */
  int32_t route_groups;   /* G: 1 = one route per chunk shared by all heads,
                             H = one route per head                            */
  natsl_dtype io;         /* dtype of x, q, k, v, out (and the decode cache)   */
  float sm_scale;         /* softmax scale; <= 0 selects 1/sqrt(Dk)            */
  float rms_eps;          /* RMSNorm epsilon (added inside the sqrt); <= 0
                             selects 1e-6                                      */
} natsl_dims;

/* Library version (major*10000 + minor*100 + patch). */
int natsl_version(void);

/* Description of the last failure on the calling thread ("" if none). */
const char* natsl_last_error(void);

/* Workspace bytes the given entry point needs for these dims (0 if none).
 * Pure host computation. */
natsl_status natsl_workspace_size(int entry, const natsl_dims* dims, size_t* bytes);

/*
 * Router (Kernmechanismen 1): for every (b, chunk c) pool x over the chunk's
 * 64 tokens (mean), score it with W_score and b_score, and pick the op with
 * the higher score (an exact tie picks softmax).  Then compact: list the
 * softmax-routed chunks per (b, g) in ascending order (the prefill form of the
 * retained softmax KV, Kernmechanismen 3).
 *   x            [B, L, d_model] io dtype (may be NULL when route_in is given)
 *   w_score      [d_model, 2G] fp32; columns (2g, 2g+1) = (softmax, linear)
 *   b_score      [2G] fp32 or NULL (zero bias)
 *   route_in     [B, G, Nc] int32 or NULL: forced routes (skips scoring)
 *   route_out    [B, G, Nc] int32   (may alias route_in)
 *   sel_idx      [B, G, Nc] int32   ascending softmax chunk ids, -1 padded
 *   nsel_before  [B, G, Nc+1] int32 softmax chunks before chunk c (exclusive)
 *   scores       [B, G, Nc, 2] fp32 or NULL
 * Reduction order is fixed, so routes are deterministic.
 */
natsl_status natsl_route(const natsl_dims* dims, const void* x, const float* w_score,
                         const float* b_score, const int32_t* route_in, int32_t* route_out,
                         int32_t* sel_idx, int32_t* nsel_before, float* scores,
                         hipStream_t stream);

/*
 * Gated DeltaNet branch with per-chunk rollback (Kernmechanismen 3): the
 * gated delta rule S_t = a_t (S_{t-1} - b_t k_t (k_t^T S_{t-1})) + b_t k_t v_t^T,
 * o_t = S_t^T q_t, pseudo-updated through every chunk; the state is carried
 * past a chunk only when route == linear, otherwise it returns to the chunk
 * start.  Computed chunkwise (UT transform per chunk, then a state scan).
 *   q, k         [B, H, L, Dk] io dtype;  v [B, H, L, Dv] io dtype
 *   alpha, beta  [B, H, L] fp32 (decay in (0, 1], write strength)
 *   route        [B, G, Nc] int32
 *   S_init       [B, H, Dk, Dv] fp32 key-major, or NULL (zero state)
 *   o_gdn        [B, H, L, Dv] of o_dtype
 *   S_final      [B, H, Dk, Dv] fp32 carried state after the last chunk, or NULL
 *   ws           workspace of natsl_workspace_size(NATSL_ENTRY_GDN_CHUNK)
 */
natsl_status natsl_gdn_chunk(const natsl_dims* dims, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const int32_t* route,
                             const float* S_init, void* o_gdn, natsl_dtype o_dtype,
                             float* S_final, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Softmax branch (Kernmechanismen 3): causal softmax attention in which a
 * query of chunk c sees the tokens of the softmax-routed chunks before c plus
 * the causal prefix of chunk c itself (whatever chunk c's own route is).
 *   q, k [B, H, L, Dk], v [B, H, L, Dv] io dtype
 *   sel_idx, nsel_before  as produced by natsl_route
 *   o_sm [B, H, L, Dv] of o_dtype
 *   lse  [B, H, L] fp32 natural-log logsumexp of the scaled scores, or NULL
 * No workspace is needed (ws may be NULL, ws_bytes 0).
 */
natsl_status natsl_softmax_masked(const natsl_dims* dims, const void* q, const void* k,
                                  const void* v, const int32_t* sel_idx,
                                  const int32_t* nsel_before, void* o_sm, natsl_dtype o_dtype,
                                  float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gradient of the softmax branch (the pages define the forward,
 * Kernmechanismen 3; this is its exact derivative).  For the keys each query
 * sees in natsl_softmax_masked, with p = exp(scale q.k - lse) and
 * delta = rowsum(d_o * o_sm):
 *   dq = scale sum_k p (d_o.v_k - delta) k,   dk = scale sum_q p (d_o.v - delta) q,
 *   dv = sum_q p d_o.
 *   q, k, v        [B, H, L, Dk] io dtype (the forward's inputs)
 *   sel_idx, nsel_before  the forward's compaction (natsl_route)
 *   o_sm           [B, H, L, Dv] io dtype: the forward's softmax branch output
 *   lse            [B, H, L] fp32: the forward's natural-log logsumexp of the
 *                  scaled scores (natsl_softmax_masked with lse)
 *   d_o            [B, H, L, Dv] io dtype: gradient of the loss w.r.t. o_sm
 *   dq, dk, dv     [B, H, L, D] fp32 outputs (written, not accumulated)
 *   dgate          [B, H, Nc] fp32 or NULL: the derivative with respect to each
 *                  chunk's softmax gate (see natsl_route_backward): with
 *                  p~ = exp(scale q.k - lse) over every key of chunk c, visible
 *                  or not, dgate[c] = sum over the queries of later chunks and
 *                  the keys of c of p~ (d_o.v - delta).  Requesting it makes a
 *                  linear-routed chunk visit the later query chunks too.
 *   ws             workspace of natsl_workspace_size(NATSL_ENTRY_SOFTMAX_BACKWARD)
 */
natsl_status natsl_softmax_masked_backward(const natsl_dims* dims, const void* q, const void* k, const void* v,
                                           const int32_t* sel_idx, const int32_t* nsel_before, const void* o_sm,
                                           const float* lse, const void* d_o, float* dq, float* dk, float* dv,
                                           float* dgate, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gradient of the Gated DeltaNet branch through the per-chunk rollback (the
 * pages define the forward, Kernmechanismen 3; this is its exact derivative).
 * The forward is natsl_gdn_chunk's: S_t = alpha_t (S_{t-1} - beta_t k_t k_t^T
 * S_{t-1}) + beta_t k_t v_t^T, o_t = S_t^T q_t, and a chunk keeps its end state
 * only when linear-routed.  Taken in chunk form: with the chunk form U = T
 * (diag(beta) V - diag(beta gamma) K S0), O = diag(gamma) Q S0 + P U, S_end =
 * gamma_C S0 + K~^T U, the carried state's gradient Gc runs backward over the
 * chunks (Gc <- [linear ? gamma_C : 1] Gc + Q^T diag(gamma) dO - W^T dU, dU =
 * P^T dO + [linear] K~ Gc), then each chunk's token gradients follow from its
 * start state S0, U, Gc and dU through T, A, P and the decays.
 *   q, k, v        [B, H, L, D] io dtype, alpha, beta [B, H, L] fp32, route
 *                  [B, G, Nc] int32 (0 softmax, 1 linear): the forward's inputs;
 *                  alpha in (0, 1] (d alpha is d log alpha / alpha)
 *   S_init         [B, H, Dk, Dv] fp32 initial state, or NULL (zeros)
 *   d_o            [B, H, L, Dv] fp32: gradient of the loss w.r.t. o_gdn
 *   dS_final       [B, H, Dk, Dv] fp32 gradient w.r.t. the final carried state,
 *                  or NULL (zeros)
 *   dq, dk, dv     [B, H, L, D] fp32 outputs; dalpha, dbeta [B, H, L] fp32
 *   dS_init        [B, H, Dk, Dv] fp32 gradient w.r.t. S_init, or NULL
 *   dgate          [B, H, Nc] fp32 or NULL: the derivative with respect to each
 *                  chunk's linear gate (see natsl_route_backward; the carried
 *                  state after chunk c written S_start + h (S_end - S_start)):
 *                  <d loss / d carried state after c, S_end - S_start>
 *   ws             workspace of natsl_workspace_size(NATSL_ENTRY_GDN_BACKWARD):
 *                  every chunk's S0 and U in the io dtype, then one region
 *                  used in turn by the forward chunk prep and by the backward
 *                  prep's output plus every chunk's Gc (about 0.88 GB for
 *                  B = 1, H = 16, L = 32768, D = 128 bf16).  A workspace of at
 *                  least natsl_workspace_size(NATSL_ENTRY_GDN_BACKWARD_OVERLAP)
 *                  (about 1.35 GB there) gives the two uses regions of their
 *                  own, and the call then runs the forward's state scan and
 *                  the reverse scan at the same time on a library helper
 *                  stream (forked from and joined back into `stream` within
 *                  the call); the results are bit-identical either way
 * Every output is written, not accumulated; results are deterministic.  The
 * matrix products take io-dtype operands (bf16 for bf16 io) with fp32
 * accumulation.  The bf16 D = 128 form has natsl_gdn_chunk's sequence-length
 * limit (NATSL_ERR_UNSUPPORTED before anything is enqueued).
 */
natsl_status natsl_gdn_backward(const natsl_dims* dims, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const int32_t* route, const float* S_init,
                                const float* d_o, const float* dS_final, float* dq, float* dk, float* dv,
                                float* dalpha, float* dbeta, float* dS_init, float* dgate, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * Gradient of the router ("Technische Samenvatting: Neural Attention Search
 * Linear (NAtS-L)", Kernmechanismen 5: the operation selection is learned end
 * to end, with gradients computed for the attention score layer; the pages do
 * not say how the argmax is differentiated).  This library's reading is the
 * straight-through estimator: the route of chunk c enters the layer as a
 * one-hot gate h_c = onehot(argmax s_c) -- the softmax branch weights chunk
 * c's keys by h_c[softmax] for the queries of later chunks, the Gated DeltaNet
 * branch commits chunk c's end state with weight h_c[linear], which at one-hot
 * h is exactly the routed forward -- and d h_c / d s_c is taken to be the
 * Jacobian of softmax(s_c).  With dh = (dgate_sm, dgate_lin) summed over the
 * heads of each route group and pi = softmax(s_c):
 *   ds = pi (dh - pi . dh);  dW[:, 2g + o] = sum_{b, c} mean_c(x) ds[b, g, c, o];
 *   db = sum ds;  dx_t = W ds_{c(t)} / 64.
 *   dims          B, H, L, d_model, route_groups, io (x's dtype)
 *   x             [B, L, d_model] io dtype;  w_score [d_model, 2G] fp32
 *   scores        [B, G, Nc, 2] fp32: the forward's scores (natsl_route /
 *                 natsl_forward scores_out)
 *   dgate_sm, dgate_lin  [B, H, Nc] fp32 (natsl_softmax_masked_backward and
 *                 natsl_gdn_backward with dgate)
 *   dx            [B, L, d_model] fp32 or NULL;  dw_score [d_model, 2G] fp32;
 *   db_score      [2G] fp32 or NULL (all written, not accumulated)
 *   ws            workspace of natsl_workspace_size(NATSL_ENTRY_ROUTE_BACKWARD)
 * Sums run in a fixed order (deterministic).  Errors as for natsl_route.
 */
natsl_status natsl_route_backward(const natsl_dims* dims, const void* x, const float* w_score, const float* scores,
                                  const float* dgate_sm, const float* dgate_lin, float* dx, float* dw_score,
                                  float* db_score, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gradient of the output merging (Kernmechanismen 4 defines the forward; this
 * is its exact derivative).  With r_x = (mean(o_x^2) + eps)^(-1/2),
 * n_x = o_x r_x g_x and (w_sm, w_lin) = softmax(q W_mix):
 *   dn_x = w_x d_out,  dw_x = d_out . n_x,  dz_sm = w_sm w_lin (dw_sm - dw_lin) = -dz_lin
 *   d_o_x = r_x u - (r_x^3 / Dv) o_x (u . o_x) with u = dn_x g_x
 *   dq = dz_sm (W_mix[:, 0] - W_mix[:, 1])   (the mixing weights' share of q's gradient)
 *   dW_mix[:, 0] = sum_t q dz_sm = -dW_mix[:, 1],   dg_x = sum_t dn_x o_x r_x
 *   q [B, H, L, Dk] io dtype, o_sm, o_gdn [B, H, L, Dv] of branch_dtype, w_mix,
 *   w_mix_head_stride, g_sm, g_lin (NULL = ones) as in natsl_merge
 *   d_out          [B, H, L, Dv] fp32: gradient of the loss w.r.t. out
 *   d_o_sm, d_o_gdn, dq  [B, H, L, D] fp32 outputs
 *   dw_mix         the shape of w_mix, fp32, or NULL; sums over all heads when
 *                  W_mix is shared (head stride 0)
 *   dg_sm, dg_lin  [Dv] fp32 (gradients of the gains, also when they are NULL
 *                  = ones), or NULL
 *   ws             workspace of natsl_workspace_size(NATSL_ENTRY_MERGE_BACKWARD)
 * Sums over tokens are added in a fixed order: results are deterministic.
 */
natsl_status natsl_merge_backward(const natsl_dims* dims, const void* q, const void* o_sm, const void* o_gdn,
                                  natsl_dtype branch_dtype, const float* w_mix, int64_t w_mix_head_stride,
                                  const float* g_sm, const float* g_lin, const float* d_out, float* d_o_sm,
                                  float* d_o_gdn, float* dq, float* dw_mix, float* dg_sm, float* dg_lin, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * Output merging (Kernmechanismen 4): per (b, h, t)
 *   n_x = o_x / sqrt(mean(o_x^2) + eps) * g_x      for x in {sm, lin}
 *   (w_sm, w_lin) = softmax(q_t . W_mix[:, 0], q_t . W_mix[:, 1])
 *   out = w_sm * n_sm + w_lin * n_lin
 *   q [B, H, L, Dk] io dtype; o_sm, o_gdn [B, H, L, Dv] branch_dtype
 *   w_mix [Dk, 2] fp32 (+ h * w_mix_head_stride floats for head h;
 *         stride 0 = shared by all heads)
 *   g_sm, g_lin [Dv] fp32 or NULL (ones);  out [B, H, L, Dv] io dtype
 */
natsl_status natsl_merge(const natsl_dims* dims, const void* q, const void* o_sm, const void* o_gdn,
                         natsl_dtype branch_dtype, const float* w_mix, int64_t w_mix_head_stride,
                         const float* g_sm, const float* g_lin, void* out, hipStream_t stream);

typedef struct {
  void* k_cache;               /* [B, H, cap, Dk] io: compacted KV             */
  void* v_cache;               /* [B, H, cap, Dv] io                           */
  int32_t cap;                 /* rows per (b, h)                              */
  int32_t* n_committed;        /* [B, G] rows of committed softmax chunks      */
  int32_t* n_open;             /* [B] tokens of the open (incomplete) chunk    */
  float* S_carry;              /* [B, H, Dk, Dv] state after committed chunks  */
  float* S_work;               /* [B, H, Dk, Dv] open chunk's pseudo-updated   */
  float* x_sum;                /* [B, d_model] sum of x over the open chunk    */
  int32_t* err_flag;           /* [1]: set to 1 when a row would exceed cap    */
} natsl_decode_cache;

typedef struct {
  const void* x;               /* [B, L, d_model] io (NULL if route_override) */
  const void* q;               /* [B, H, L, Dk] io                            */
  const void* k;               /* [B, H, L, Dk] io                            */
  const void* v;               /* [B, H, L, Dv] io                            */
  const float* alpha;          /* [B, H, L]                                   */
  const float* beta;           /* [B, H, L]                                   */
  const float* w_score;        /* [d_model, 2G] (NULL if route_override)      */
  const float* b_score;        /* [2G] or NULL                                */
  const float* w_mix;          /* [Dk, 2] (+ head stride)                     */
  int64_t w_mix_head_stride;   /* 0 = shared                                  */
  const float* g_sm;           /* [Dv] or NULL                                */
  const float* g_lin;          /* [Dv] or NULL                                */
  const int32_t* route_override; /* [B, G, Nc] or NULL                        */
  const float* S_init;         /* [B, H, Dk, Dv] or NULL                      */
  natsl_dtype branch_dtype;    /* dtype of the intermediate branch outputs    */
  int32_t* route_out;          /* [B, G, Nc] or NULL                          */
  float* scores_out;           /* [B, G, Nc, 2] or NULL                       */
  void* o_sm_dbg;              /* [B, H, L, Dv] branch_dtype or NULL: raw
                                  softmax branch output                       */
  void* o_gdn_dbg;             /* [B, H, L, Dv] branch_dtype or NULL: raw
                                  Gated DeltaNet branch output                */
  float* S_final;              /* [B, H, Dk, Dv] or NULL                      */
  void* out;                   /* [B, H, L, Dv] io                            */
  const natsl_decode_cache* prefix; /* NULL, or the decode cache this segment
                                  continues (chunked prefill, see below)      */
} natsl_forward_args;

/*
 * Whole layer forward ("Technische Samenvatting: Neural Attention Search
 * Linear (NAtS-L)", Kernmechanismen 1-4): route + compaction (item 1), the
 * Gated DeltaNet branch with per-chunk rollback and the softmax branch over
 * the retained softmax chunks plus the own chunk (item 3; run concurrently),
 * then RMSNorm of both outputs and the Q-derived weighted sum (item 4).
 * Every pointer of args is a device pointer as documented in the struct; x
 * and w_score may be NULL only with route_override.  Outputs: out always;
 * route_out, scores_out (router only), o_sm_dbg, o_gdn_dbg, S_final when
 * non-NULL.  ws from NATSL_ENTRY_FORWARD (caller-owned, >= that size, 256-byte
 * aligned); the call reads and writes it until the work it enqueues on
 * `stream` has finished.  Errors: NATSL_ERR_INVALID_ARG (NULL input, bad
 * dtype or stride, S_init together with a prefix), NATSL_ERR_UNSUPPORTED
 * (dims), NATSL_ERR_WORKSPACE, all before anything is enqueued;
 * NATSL_ERR_DEVICE for a failed HIP call (the helper stream is still joined).
 * Chunked prefill: with args->prefix set, the L tokens are a segment that
 * continues that decode cache, which must sit at a chunk boundary
 * (n_open == 0, e.g. right after natsl_decode_handoff): every query of the
 * segment also attends to the cache's min(n_committed, cap) committed softmax
 * rows (before the segment's own chunks), and the Gated DeltaNet branch starts
 * from the cache's S_carry (S_init must then be NULL).  The outputs equal
 * those of one prefill over the cached prefix and the segment; appending the
 * segment with natsl_decode_handoff(..., append = 1) then gives the cache of
 * that whole prefill.  The prefix is only read.
 */
natsl_status natsl_forward(const natsl_dims* dims, const natsl_forward_args* args, void* ws,
                           size_t ws_bytes, hipStream_t stream);


typedef struct {
  const void* x;               /* [B, d_model] io                              */
  const void* q;               /* [B, H, Dk] io                                */
  const void* k;               /* [B, H, Dk] io                                */
  const void* v;               /* [B, H, Dv] io                                */
  const float* alpha;          /* [B, H]                                       */
  const float* beta;           /* [B, H]                                       */
  const float* w_score;        /* [d_model, 2G]                                */
  const float* b_score;        /* [2G] or NULL                                 */
  const float* w_mix;          /* [Dk, 2] (+ head stride)                      */
  int64_t w_mix_head_stride;
  const float* g_sm;           /* [Dv] or NULL                                 */
  const float* g_lin;          /* [Dv] or NULL                                 */
  void* out;                   /* [B, H, Dv] io                                */
  int32_t* route_out;          /* [B, G] or NULL: -1 no chunk completed this
                                  step, else the completed chunk's route       */
  float* o_sm_dbg;             /* [B, H, Dv] fp32 or NULL                      */
  float* o_gdn_dbg;            /* [B, H, Dv] fp32 or NULL                      */
} natsl_decode_args;

/*
 * One decode step ("Technische Samenvatting: Neural Attention Search Linear
 * (NAtS-L)", Kernmechanismen 1, 3 and 4 applied one token at a time: the two
 * hidden states are the retained softmax KV and the Gated DeltaNet state;
 * the chunk's operation is chosen when the chunk is complete, and only the
 * chosen operation keeps it).  Every sequence appends one token to its open
 * chunk.  Softmax over the committed softmax chunks' rows, the open chunk's
 * earlier rows and the new token; the Gated DeltaNet state is pseudo-updated
 * from S_carry (first token of a chunk) or S_work.  When the open chunk
 * reaches 64 tokens it is routed from x_sum / 64: softmax commits its 64
 * rows (n_committed += 64), linear commits its state (S_carry <- S_work) and
 * its rows are dropped.  The cache (natsl_decode_cache) is read and updated
 * in place on the device; args' tensors are read, out / route_out / the dbg
 * outputs written.  Errors: NATSL_ERR_INVALID_ARG (NULL tensor, cap < 1),
 * NATSL_ERR_UNSUPPORTED (dims; cap above 2^30; B * H * ceil(cap / 1024) at
 * or above 2^24, the attention's workgroup count), NATSL_ERR_WORKSPACE, all before anything is
 * enqueued; NATSL_ERR_DEVICE for a failed launch.  The new row is written at index n_committed + n_open;
 * if that index is >= cap the row is not written and *err_flag is set to 1
 * (checked by the caller after the step; counters still advance).
 * ws from NATSL_ENTRY_DECODE_STEP (depends on cap via dims->L: pass
 * dims->L = cap).
 */
natsl_status natsl_decode_step(const natsl_dims* dims, const natsl_decode_cache* cache,
                               const natsl_decode_args* args, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Scratch the allocation-free decode step holds per device (bytes). */
#define NATSL_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * Allocation-free decode step, for callers that cannot allocate device
 * memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The same step, arguments
 * and errors as natsl_decode_step without ws / ws_bytes: the step's scratch
 * (per-sequence chunk decisions, the Gated DeltaNet outputs, the split-KV
 * partials) lives in a NATSL_DECODE_NOALLOC_SCRATCH_BYTES array that the
 * library keeps in each device's memory until the process ends; the call
 * itself allocates nothing.  Dims whose natsl_workspace_size(
 * NATSL_ENTRY_DECODE_STEP) exceeds that size are NATSL_ERR_WORKSPACE, before
 * anything is enqueued (e.g. B = 64, H = 16, D = 128 takes caches of up to
 * about 28,000 rows).  Every call on one device uses that device's array and
 * leaves its contents behind (each step writes every scratch value it later
 * reads, so nothing needs clearing): two calls whose work can overlap on one
 * device (different streams with no ordering between them) race on it and
 * must be ordered by the caller.
 */
natsl_status natsl_decode_step_noalloc(const natsl_dims* dims, const natsl_decode_cache* cache,
                                       const natsl_decode_args* args, hipStream_t stream);

/*
 * Prefill -> decode handoff ("Technische Samenvatting: Neural Attention Search
 * Linear (NAtS-L)", Kernmechanismen 3: the softmax operation keeps only the KV
 * of the chunks routed to it, the linear operation its fixed-size state).
 * Fills `cache` as a decode continuing after a prefill of dims->L tokens
 * (L % 64 == 0) expects it:
 *   k_cache/v_cache rows [0, 64 * n) of (b, h) = the K/V rows of the n
 *     softmax-routed chunks of (b, g(h)), in chunk order (bit copies); rows
 *     from 64 * n on are left as they were;
 *   n_committed[b, g] = 64 * n;  n_open[b] = 0;
 *   S_carry = S_final (the state natsl_forward returns) or zero when S_final
 *     is NULL;  S_work = 0;  x_sum = 0;
 *   *err_flag = 0, or 1 when some 64 * n exceeds cap (the rows at or beyond
 *     cap are not written; n_committed still counts them).
 *   dims      B, H, L, Dk (= Dv), route_groups G, d_model, io of the prefill
 *   route     [B, G, L/64] int32, 0 = softmax, 1 = linear (route_out of
 *             natsl_forward or natsl_route)
 *   k, v      [B, H, L, Dk] io dtype: the prefill's keys and values
 *   S_final   [B, H, Dk, Dv] fp32 or NULL
 *   cache     its tensors as in natsl_decode_step, cap = its capacity
 *   append    0: as above.  1: the cache already holds a prefix at a chunk
 *             boundary and the L tokens were a segment prefilled on top of it
 *             (natsl_forward with args->prefix = cache): the segment's softmax
 *             rows go to rows [n_committed, n_committed + 64 n) and
 *             n_committed += 64 n; S_carry = S_final (required); S_work,
 *             x_sum, n_open as above; *err_flag is not cleared, and is set
 *             when a row would reach cap or the cache has an open chunk.
 *   ws        workspace of natsl_workspace_size(NATSL_ENTRY_DECODE_HANDOFF)
 * A prefix whose last chunk is incomplete continues with natsl_decode_step
 * for its remaining tokens: the route of an incomplete chunk affects no
 * prefill output, so that gives the same outputs and cache.
 */
natsl_status natsl_decode_handoff(const natsl_dims* dims, const int32_t* route, const void* k, const void* v,
                                  const float* S_final, int append, const natsl_decode_cache* cache, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * Native Hybrid Attention ("Native Hybrid Attention for Efficient Sequence
 * Modeling", section 2 Methodologie, "Unificatie van Intra-layer
 * Hybridisatie"): long-term information is compressed into `slots` key-value
 * slots by a linear RNN update, the slots are joined with the tokens of a
 * sliding window into one key-value set, and one softmax attention runs over
 * that set (window 0: the slots alone, a linear RNN; a window covering the
 * sequence: causal softmax attention).  The page gives no equations; this
 * library's reading:
 *   - query t sees the keys and values of tokens t-window+1 .. t;
 *   - token s enters the slots when it leaves the window (before query
 *     s + window), per slot i with its gate a_s[i] in [0, 1]:
 *       K~[i] <- a_s[i] K~[i] + (1 - a_s[i]) k_s,  V~[i] likewise;
 *     slots start at zero and join the key set once a token has entered;
 *   - scores scale * q_t . key (scale: dims->sm_scale, <= 0 = 1/sqrt(Dk)).
 *   dims        B, H, L, Dk = Dv in {64, 128}, io (L % 64 == 0; route_groups,
 *               d_model unused)
 *   q, k, v     [B, H, L, D] io dtype
 *   slot_gate   [B, H, L, slots] fp32, the gate of each token for each slot
 *   slots       16, 32 or 64
 *   window      tokens, a multiple of 64 (>= L: plain causal attention)
 *   out         [B, H, L, D] io dtype
 *   ws          natsl_nha_workspace_size bytes (the slots' states at every
 *               chunk start and the window's partial result, fp32)
 * The window's softmax runs on the helper stream beside the slot-state
 * kernels (it needs none of them) and is joined before the slots' read-out.
 * Errors: NATSL_ERR_UNSUPPORTED (slots, window or dims), NATSL_ERR_INVALID_ARG,
 * NATSL_ERR_WORKSPACE, before anything is enqueued; NATSL_ERR_DEVICE.
 */
natsl_status natsl_nha_workspace_size(const natsl_dims* dims, int slots, int window, size_t* bytes);
natsl_status natsl_nha_attention(const natsl_dims* dims, const void* q, const void* k, const void* v,
                                 const float* slot_gate, int slots, int window, void* out, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/*
 * Synchronous-check debug mode (not part of the method; for finding which call
 * raised a device error).  level 0: off (the default).  level 1: every entry
 * point that enqueues work waits for `stream` before it returns, and the first
 * error the HIP runtime reports there becomes NATSL_ERR_DEVICE whose message
 * names the entry point.  level 2: as 1, and the entry point's name is written
 * to stderr (flushed) before the wait, so that a fault which ends the process
 * still names the call.  A stream under graph capture is never waited for.
 * Without a call to natsl_set_sync_check the level is read once, at the first
 * call that needs it, from the environment variable NATSL_SYNC_CHECK ("1" or
 * "2"; unset, empty or "0" is off).  The level is process-wide; calls on other
 * threads see a change at their next entry.  natsl_set_sync_check returns
 * NATSL_ERR_INVALID_ARG for a level outside 0..2 and changes nothing then.
 */
natsl_status natsl_set_sync_check(int level);
int natsl_get_sync_check(void);

/*
 * Kernel timing for measurement: when enabled, every kernel the library
 * launches is bracketed by HIP events on the stream it runs on.
 * natsl_profile_read synchronises those events and returns, for the kernel
 * named `name`, the number of recorded launches and their summed duration
 * in milliseconds since the last reset.  Names: "route", "compact",
 * "gdn_prep", "gdn_scan", "softmax_masked", "merge", "decode_route",
 * "decode_gdn", "decode_attn", "decode_combine", "decode_commit",
 * "softmax_backward", "decode_handoff", "gdn_backward", "merge_backward",
 * "route_backward", "nha" (each a whole call of that entry) and "nha_window",
 * "nha_chunk", "nha_scan", "nha_slots" (the kernels of natsl_nha_attention).
 * natsl_profile_select restricts the recording to the kernel named `name`
 * (NULL or "" records every kernel again), so that timing one kernel adds
 * only its own two event records to a step; an unknown name is
 * NATSL_ERR_INVALID_ARG and leaves the selection unchanged.
 */
natsl_status natsl_profile_enable(int on);
natsl_status natsl_profile_reset(void);
natsl_status natsl_profile_read(const char* name, int* count, double* total_ms);
natsl_status natsl_profile_select(const char* name);

#ifdef __cplusplus
}
#endif
#endif /* NATSL_H */
