/* latentmoe.h - C ABI of the MI355X (gfx950) Stable LatentMoE forward.
 *
 * The layer (K3 notes, raw notes/sections/sec-07.tex @47c72e5, chapter
 * "SiTU-GLU and Stable LatentMoE", five-step compute flow):
 *   1. z    = W_down x                                   latent compression, width l
 *   2. s    = sigmoid(W_r x), T = TopK(s + b, k),        K3 sigmoid routing; the bias b
 *      p_i  = s_i / sum_{j in T} s_j                     only affects which experts win
 *   3. u    = sum_{i in T} p_i E_i(z)                    routed SiTU-GLU experts, width l,
 *                                                        run as permute-dispatch -> grouped
 *                                                        GEMMs -> p-weighted scatter-add
 *   4. s_sh = sum_j E_j^sh(x)                            shared SiTU-GLU experts, width d
 *   5. y    = s_sh + W_up RMSNorm(u)
 * with SiTU-GLU E(v) = W_o [beta1 tanh(W_g v / beta1) sigmoid(W_g v) * beta2 tanh(W_u v / beta2)]
 * (same chapter, SiTU-GLU equation).
 *
 * Conventions shared by every entry point
 *  - Every tensor argument is device memory allocated and owned by the caller,
 *    row-major and contiguous, 16-byte aligned.  Matrices are stored like
 *    nn.Linear weights, [out, in].
 *  - Storage type: dims->dtype selects fp32 (LMOE_F32) or bf16 (LMOE_BF16) for
 *    x, every weight matrix, the padded tensor and y.  bias, rms_w, probs,
 *    logits and u are always fp32.  Accumulation is always fp32.  In bf16 mode
 *    the intermediates that feed a second matrix product or a sum -- z, the
 *    SiTU hidden h, the p-weighted expert outputs (one row per (token, slot)
 *    pair, summed per token in slot order) and RMSNorm(u) -- are held in fp16
 *    (11-bit significand), and the bf16 weights they meet are widened to fp16
 *    (exact for |w| >= 2^-14).  Range: |h| < beta1*beta2 by the SiTU bound
 *    (bf16 storage requires beta1*beta2 < 65504), |RMSNorm(u)| <= sqrt(l) *
 *    max|rms_w|, and z = W_down x and p E(z) stay far below 65504 for
 *    unit-scale (pre-normed) x and N(0, 1/fan_in) weights.  The forward checks
 *    z, the p-weighted outputs and RMSNorm(u) as it stores them: a value that
 *    would round to inf in fp16 (or is NaN) raises a flag in the workspace,
 *    reported as LMOE_ERR_RANGE by the synchronous forward and by
 *    latentmoe_forward_check.  The backward's fp16 intermediates are not
 *    checked.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *    default stream) and is asynchronous unless an entry point says otherwise.
 *  - `workspace` is caller-owned device scratch of at least
 *    latentmoe_workspace_bytes(dims, entry) bytes; the library allocates no
 *    device memory.  Calls that share a workspace must be ordered on one
 *    stream.  The one state kept between calls: latentmoe_forward's
 *    overlapped path (n_shared > 0 and N d n_s f_s <= 2048 * 7168 * 18432, i.e.
 *    up to 2048 tokens at the full-K3 widths) creates, on first use by a
 *    host thread on a device, a second non-blocking stream of default
 *    priority for that thread and device, kept until the process ends.
 *  - Matrices (x, y, z, the padded tensor, u, du, dz, dy, dx and every weight
 *    and weight-gradient matrix) and the workspace must be 16-byte aligned, as
 *    hipMalloc and torch allocations are: they are moved 16 bytes at a time.
 *    A misaligned one is INVALID_ARGUMENT.  Vectors (ids, probs, counts, bias,
 *    logits, ...) need only their element alignment.
 *  - Errors: a status code, never an abort.  Arguments are validated before
 *    anything is enqueued; on any error the outputs are unspecified.
 *    latentmoe_last_error() returns a thread-local description of the last
 *    failure on the calling thread.
 *  - Supported shapes: d, l, f_r and f_s multiples of 64; 1 <= k <= R <= 4096,
 *    k <= 64; 0 <= n_shared <= 16; n_tokens >= 0 (0 is a no-op).
 */
#ifndef LATENTMOE_H
#define LATENTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMOE_OK = 0,
  LMOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, k < 1, k > R, non-positive width, beta <= 0, eps < 0 */
  LMOE_ERR_UNSUPPORTED = 2,      /* a shape outside the limits listed above */
  LMOE_ERR_CAPACITY = 3,         /* padded buffer too small for C (C is still reported) */
  LMOE_ERR_WORKSPACE = 4,        /* workspace smaller than latentmoe_workspace_bytes() */
  LMOE_ERR_HIP = 5,              /* a HIP runtime call or launch failed */
  LMOE_ERR_RANGE = 6             /* bf16 storage: an fp16 intermediate of the forward left fp16's
                                    range (see the conventions above); outputs unspecified */
} lmoe_status;

typedef enum { LMOE_F32 = 0, LMOE_BF16 = 1 } lmoe_dtype;

/* Which entry point a workspace size is asked for. */
typedef enum {
  LMOE_ENTRY_ROUTE = 0,
  LMOE_ENTRY_DISPATCH = 1,
  LMOE_ENTRY_EXPERTS = 2,
  LMOE_ENTRY_FORWARD = 3,
  LMOE_ENTRY_ROUTED_BACKWARD = 4,
  LMOE_ENTRY_BACKWARD = 5
} lmoe_entry;

/* Layer sizes (names after the chapter's component table). */
typedef struct {
  int64_t n_tokens;  /* N = B*T; tokens are independent, batch structure is irrelevant */
  int32_t d_model;   /* d */
  int32_t d_latent;  /* l (the chapter uses l = d/2; any multiple of 64 is accepted) */
  int32_t n_routed;  /* R */
  int32_t top_k;     /* k */
  int32_t n_shared;  /* n_s (0 allowed) */
  int32_t ff_routed; /* f_r, inner width of a routed expert */
  int32_t ff_shared; /* f_s, inner width of a shared expert (f_r == f_s gives the pages' single d_ff) */
  float beta1;       /* SiTU gate cap, 4 on the pages */
  float beta2;       /* SiTU up cap, 25 on the pages */
  float rms_eps;     /* RMSNorm eps (inside the square root) */
  int32_t dtype;     /* lmoe_dtype */
} lmoe_dims;

/* Parameters of one layer (all device pointers, storage dtype unless fp32 is stated). */
typedef struct {
  const void* w_down;   /* [l, d]          W_down */
  const void* w_router; /* [R, d]          W_r */
  const float* bias;    /* [R] fp32        expert bias b (selection only); NULL = zeros */
  const void* w_g;      /* [R, f_r, l]     routed gate projections */
  const void* w_u;      /* [R, f_r, l]     routed up projections */
  const void* w_o;      /* [R, l, f_r]     routed output projections */
  const void* sh_g;     /* [n_s, f_s, d]   shared gate projections (unused if n_s = 0) */
  const void* sh_u;     /* [n_s, f_s, d]   shared up projections */
  const void* sh_o;     /* [n_s, d, f_s]   shared output projections */
  const float* rms_w;   /* [l] fp32        RMSNorm weight; NULL = ones */
  const void* w_up;     /* [d, l]          W_up */
} lmoe_weights;

/* Gradients of the layer's parameters (device pointers, caller-owned, the
 * same shapes and dtypes as lmoe_weights; the bias gets none). */
typedef struct {
  void* w_down;   /* [l, d] */
  void* w_router; /* [R, d] */
  void* w_g;      /* [R, f_r, l] */
  void* w_u;      /* [R, f_r, l] */
  void* w_o;      /* [R, l, f_r] */
  void* sh_g;     /* [n_s, f_s, d] (unused if n_s = 0) */
  void* sh_u;     /* [n_s, f_s, d] */
  void* sh_o;     /* [n_s, d, f_s] */
  float* rms_w;   /* [l] fp32 */
  void* w_up;     /* [d, l] */
} lmoe_grads;

/* Bytes of workspace an entry point needs for these dims. */
size_t latentmoe_workspace_bytes(const lmoe_dims* dims, int32_t entry);

const char* latentmoe_status_string(lmoe_status status);
const char* latentmoe_last_error(void);

/* K3 sigmoid routing (chapter step 2 and its routing code with the three
 * notes that follow it):
 *   logits = W_r x (fp32 accumulation), s = sigmoid(logits), T = the k experts
 *   with the largest s + b (equal values: lower id first), p_i = s_i / max(sum_T s, 1e-9).
 * x [N, d] and w_router [R, d] in the storage dtype, bias [R] fp32 (NULL = zeros).
 * Outputs: ids [N, k] int32 in descending s + b order, probs [N, k] fp32 in the
 * same order, and optionally logits [N, R] fp32 (NULL to skip; the Switch
 * auxiliary and z losses are computed from them).  Asynchronous. */
lmoe_status latentmoe_route(const lmoe_dims* dims, const void* x, const void* w_router,
                            const float* bias, int32_t* ids, float* probs, float* logits,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Permute-dispatch (chapter section on sparse execution: permute-dispatch
 * + padded bmm).  The N*k (token, slot) pairs, numbered q = n*k + j, are
 * sorted stably by expert id:
 *   counts [R]   pairs per expert               offsets [R]  exclusive prefix sum of counts
 *   order [N*k]  q of the pair at each sorted position (expert-major, ascending q inside an expert)
 *   *C_out       capacity C = max counts (host int64, required)
 * If padded is not NULL, padded [R, C, l] (storage dtype, stride C, the first
 * R*C*l elements of a buffer of capacity*R*l elements) receives row
 * padded[e, r] = z[order[offsets[e] + r] / k] for r < counts[e] and zeros
 * for r >= counts[e].  If C > capacity nothing is written to padded and
 * LMOE_ERR_CAPACITY is returned with *C_out set.
 * Synchronous: waits on `stream` to read C (the pages' layout needs C on the host). */
lmoe_status latentmoe_dispatch(const lmoe_dims* dims, const int32_t* ids, const void* z,
                               int32_t* counts, int32_t* offsets, int32_t* order, void* padded,
                               int64_t capacity, int64_t* C_out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Routed SiTU-GLU experts on the padded layout (chapter step 3 and the three
 * batched products of the sparse-execution section), with the p-weighted
 * scatter-add back to token order:
 *   u[n] = sum_j probs[n, j] * E_{ids[n, j]}(z[n])
 * padded [R, C, l] as written by latentmoe_dispatch, counts/offsets/order as
 * returned by it, probs [N, k] fp32 (the router's p), w_g/w_u [R, f_r, l],
 * w_o [R, l, f_r].  Padding rows are never read.  Output u [N, l] fp32,
 * overwritten.  Asynchronous.
 * C is the row stride the padded buffer was laid out with, 1 <= C <= N.  The
 * pages take C = max counts; with a smaller C the buffer holds only each
 * expert's first C pairs, and its later pairs are dropped: they add nothing
 * to u.  No read leaves the R * C * l elements of `padded`. */
lmoe_status latentmoe_experts(const lmoe_dims* dims, const void* padded, int64_t C,
                              const int32_t* counts, const int32_t* offsets, const int32_t* order,
                              const float* probs, const void* w_g, const void* w_u,
                              const void* w_o, float* u, void* workspace, size_t workspace_bytes,
                              void* stream);

/* The whole layer, steps 1-5.  x [N, d] in, y [N, d] out (storage dtype).
 * Side outputs (the pages' route bookkeeping): ids [N, k] int32 and
 * probs [N, k] fp32 as from latentmoe_route, counts [R] int32 pairs per
 * expert.  If C_host is not NULL the call waits on `stream`, writes
 * C = max counts there and returns LMOE_ERR_RANGE if an fp16 intermediate
 * left fp16's range; with C_host NULL the call is fully asynchronous: it
 * only enqueues kernels (and, on the overlapped path, an event fork and
 * join with a second stream), so a caller may capture it in a HIP graph,
 * and latentmoe_forward_check reads the range flag afterwards.
 * The routed experts read their rows straight from z through the sorted
 * pair order (the padded tensor is not materialised), skip empty experts and
 * padding rows, and the scatter-add is deterministic (each pair writes its own
 * slot; slots are summed in slot order).  When N d n_s f_s <= 2048 * 7168 *
 * 18432 (the overlapped path: up to 2048 tokens at the full-K3 widths) the
 * shared experts' gate/up GEMM runs on a second, library-owned stream (one
 * per calling host thread and device), forked from and joined back into
 * `stream` with events (capturable as a fork/join in a HIP graph); all other
 * work is on `stream`. */
lmoe_status latentmoe_forward(const lmoe_dims* dims, const lmoe_weights* weights, const void* x,
                              void* y, int32_t* ids, float* probs, int32_t* counts,
                              int64_t* C_host, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Range status of the last latentmoe_forward (or latentmoe_forward_timed)
 * enqueued with this workspace and dims: waits on `stream`, then returns
 * LMOE_ERR_RANGE if an fp16 intermediate of that forward left fp16's range
 * (its y is then unspecified), LMOE_OK otherwise.  For callers of the
 * asynchronous form (C_host NULL), e.g. after replaying a captured forward.
 * workspace NULL (with dims that fit it): the current device's fixed scratch,
 * i.e. the last latentmoe_forward_noalloc on this device.
 * Errors: INVALID_ARGUMENT for bad dims, WORKSPACE for a short workspace. */
lmoe_status latentmoe_forward_check(const lmoe_dims* dims, const void* workspace, size_t workspace_bytes,
                                    void* stream);

/* latentmoe_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results as latentmoe_forward with C_host
 * NULL (asynchronous, launches only), minus the workspace: the intermediates
 * live in a fixed scratch array of 64 MiB that the library holds on each
 * device it runs on until the process ends (enough for the full-K3 layer
 * up to ~170 tokens, the 0.5b layer up to 4096).  All steps run on `stream`
 * (no second stream).  The call allocates nothing (no hipMalloc, no
 * library allocation); its first call on a device looks up the array's
 * address there.  Every call on one device shares that device's array:
 * calls that overlap in time on one device (other streams, other threads)
 * race and must be ordered by the caller.  The range flag is read with
 * latentmoe_forward_check(dims, NULL, 0, stream).  Errors: as
 * latentmoe_forward, and LMOE_ERR_WORKSPACE when the dims need more scratch
 * than the array holds (nothing is enqueued). */
lmoe_status latentmoe_forward_noalloc(const lmoe_dims* dims, const lmoe_weights* weights, const void* x,
                                      void* y, int32_t* ids, float* probs, int32_t* counts, void* stream);

/* Backward of the routed-expert block u = sum_j p_j E_{ids_j}(z) (chapter
 * step 3 and the sparse-execution section, differentiated; the pages train
 * this layer and their tests compare its sparse gradients with the dense
 * helper's) for an upstream gradient du = dL/du.  Per pair (n, j), e = ids[n, j]:
 *   a_g = W_g^e z_n, a_u = W_u^e z_n, h = SiTU hidden, o = W_o^e h
 *   dprobs[n, j] = <du_n, o>          dW_o^e += p du_n h^T
 *   g_h = (W_o^e)^T (p du_n), g_g = g_h * dh/da_g, g_u = g_h * dh/da_u
 *   dW_g^e += g_g z_n^T, dW_u^e += g_u z_n^T, dz_n += (W_g^e)^T g_g + (W_u^e)^T g_u
 * Inputs: z [N, l] and the weights w_g, w_u [R, f_r, l], w_o [R, l, f_r] in the
 * storage dtype; ids [N, k] int32 and probs [N, k] fp32 as from
 * latentmoe_route; du [N, l] fp32.  Outputs (device memory, caller-owned):
 * dz [N, l] fp32, dprobs [N, k] fp32, dw_g, dw_u [R, f_r, l] and dw_o
 * [R, l, f_r] in the storage dtype (fp32 accumulation, one rounding); every
 * expert without pairs gets exact zeros.  With bf16 storage the pair
 * intermediates are fp16 (as in the forward).  The pre-activations are
 * recomputed from z.  Reads C back (waits on `stream` once); the rest is
 * asynchronous.  Workspace: latentmoe_workspace_bytes(dims,
 * LMOE_ENTRY_ROUTED_BACKWARD) bytes of device memory (the recomputed pair
 * quantities and per-expert transposed pair blocks; with fp32 storage also
 * transposed copies of the routed weights, 16-bit weights are read as stored).
 * Errors: INVALID_ARGUMENT for bad dims, NULL
 * pointers or ids outside [0, R); WORKSPACE. */
lmoe_status latentmoe_routed_backward(const lmoe_dims* dims, const void* z, const int32_t* ids,
                                      const float* probs, const void* w_g, const void* w_u,
                                      const void* w_o, const float* du, float* dz, float* dprobs,
                                      void* dw_g, void* dw_u, void* dw_o, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Backward of the whole layer (the five compute-flow steps differentiated in
 * reverse order, routes held fixed: top-k is piecewise constant and the bias
 * only selects) for an upstream gradient dy = dL/dy:
 *   5. dW_up = dy^T r, dr = dy W_up; r = RMSNorm(u) -> du, drms_w
 *   4. dS_o^j = dy^T h_j; through SiTU: dS_g^j, dS_u^j, dx += g_g S_g^j + g_u S_u^j
 *   3. the routed block as in latentmoe_routed_backward -> dz, dprobs, dW_g, dW_u, dW_o
 *   2. ds = (dp - sum_T p dp) / sum_T s on the selected experts, dl = ds s (1 - s),
 *      dW_r = dl^T x, dx += dl W_r
 *   1. dW_down = dz^T x, dx += dz W_down
 * Inputs: x [N, d] and dy [N, d] in the storage dtype; ids [N, k] and probs
 * [N, k] as returned by latentmoe_forward for this x.  Outputs: dx [N, d]
 * fp32 and every parameter gradient in `grads` (storage dtype, rms_w fp32;
 * fp32 accumulation, one rounding).  The forward quantities (z, u, the shared
 * pre-activations) are recomputed; u is formed as the forward forms it (the
 * p-weighted expert outputs held in the intermediate type, summed in slot
 * order).  Reads C back once; otherwise
 * asynchronous.  Workspace: latentmoe_workspace_bytes(dims,
 * LMOE_ENTRY_BACKWARD) bytes of device memory.  Errors: INVALID_ARGUMENT for
 * bad dims, NULL pointers or ids outside [0, R); WORKSPACE. */
lmoe_status latentmoe_backward(const lmoe_dims* dims, const lmoe_weights* weights, const void* x,
                               const int32_t* ids, const float* probs, const void* dy, float* dx,
                               const lmoe_grads* grads, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Legacy router that the K3 sigmoid router replaced (compare page, forward
 * hunk of latent_moe.py): ids = the k largest raw logits = W_r x (equal values:
 * lower id first), probs = softmax over those k logits.  Arguments as for
 * latentmoe_route, without a bias.  Asynchronous. */
lmoe_status latentmoe_route_softmax(const lmoe_dims* dims, const void* x, const void* w_router,
                                    int32_t* ids, float* probs, float* logits, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Switch/GShard auxiliary loss and router z-loss (chapter section on load
 * balancing), unscaled (the layer multiplies them by its coefficients):
 *   f_e = counts_e / sum_e counts_e,  P_e = mean over tokens of sigmoid(l_te),
 *   out[0] = R * sum_e f_e P_e,      out[1] = mean over tokens of (logsumexp_e l_te)^2.
 * logits [N, R] fp32 as written by latentmoe_route; counts [R] int32 (from
 * latentmoe_dispatch or latentmoe_forward); out: 2 fp32 in device memory.
 * N = 0 gives {0, 0}.  Deterministic (fixed summation order).  Workspace:
 * latentmoe_router_losses_workspace_bytes(dims) bytes of device memory, owned
 * by the caller.  Errors: INVALID_ARGUMENT for bad dims or a NULL pointer,
 * WORKSPACE when it is missing or too small.  Asynchronous. */
size_t latentmoe_router_losses_workspace_bytes(const lmoe_dims* dims);
lmoe_status latentmoe_router_losses(const lmoe_dims* dims, const float* logits, const int32_t* counts,
                                    float* out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* latentmoe_forward with timing marks, for profiling: `events` holds
 * LMOE_FORWARD_TIMING_EVENTS hipEvent_t handles (created by the caller);
 * events[0] is recorded on `stream` before the first step and events[i]
 * after step i, in this order:
 *   1 latent compression GEMM         5 routed gate/up grouped GEMM (+ tile list)
 *   2 router logits GEMM + top-k      6 routed down grouped GEMM -> slots
 *   3 dispatch (hist, scan, scatter)  7 slot sum + RMSNorm
 *   4 shared gate/up GEMM             8 merge GEMM [h_shared | RMSNorm(u)] -> y
 * The elapsed time between events[i-1] and events[i] is step i's device time.
 * All steps run in order on `stream` (latentmoe_forward, on its overlapped path,
 * runs step 4 on a second stream of its own next to steps 1-3 and 5-7).  C is
 * not read back.  Otherwise identical to latentmoe_forward. */
#define LMOE_FORWARD_TIMING_EVENTS 9
lmoe_status latentmoe_forward_timed(const lmoe_dims* dims, const lmoe_weights* weights,
                                    const void* x, void* y, int32_t* ids, float* probs,
                                    int32_t* counts, void* workspace, size_t workspace_bytes,
                                    void* stream, void* const* events, int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* LATENTMOE_H */
