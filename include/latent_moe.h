/*
 * latent_moe.h — C ABI of the MI355X (gfx950) LatentMoE feed-forward layer.
 *
 * The layer (vLLM Kimi K3 post, "Kimi K3 Inference Backend Evolution", section
 * 1 "LatentMoE: Dimensionality Reduction at the Routing Inlet, Restoration at
 * the Outlet"; TokenSpeed AgentX post, "Model architecture"):
 *
 *   z    = x W_in^T                              latent down-projection [T,l]
 *   ids, w = top-k of E router logits, softmax over the k                 [T,k]
 *                                                (logits given, or computed
 *                                                as z W_router^T: see
 *                                                latent_moe_layer)
 *   H    = silu(z W1_e^T) * (z W3_e^T)           routed SwiGLU expert, in latent
 *   Y    = H W2_e^T                              per (token, slot) row
 *   c    = sum_j w[t,j] Y[t,j]                   weighted combine (fp32)
 *   rhat = c / sqrt(mean(c^2) + eps) * gain      routed-latent RMSNorm (optional;
 *                                                vLLM post section 6 "Latent MoE
 *                                                Tail"; TokenSpeed Day-0 post,
 *                                                "Iris and communication")
 *   hs   = silu(x Ws1^T) * (x Ws3^T)             S shared experts, hidden width
 *   y    = rhat W_out^T + hs Ws2^T               latent up-projection + shared
 *
 * bf16 storage (round to nearest even) at z, H, Y, rhat, hs and y; every
 * GEMM accumulates in fp32.  MXFP4 expert weights (OCP MX v1.0 e2m1 + one
 * e8m0 scale per 32 along K) run either "w4a8" (TokenSpeed Day-0 post,
 * "TensorRT-LLM Stable LatentMoE"): activations entering each expert GEMM are
 * quantised to MXFP8 (e4m3fn + e8m0 per 32) and multiplied on CDNA4's
 * block-scaled MFMA; or "w4a16": bf16 activations times the exactly upcast
 * weights on bf16 MFMAs (see the LMOE_WFMT_* values below).
 *
 * Conventions shared by every call
 *  - All tensors are row-major and contiguous; weights are [out, in] (the
 *    reduction dimension is the contiguous one).  bf16 is passed as its 16-bit
 *    pattern (void*).  Every device pointer must be 16-byte aligned.
 *  - Device buffers (inputs, outputs, workspaces) are owned by the caller; the
 *    library never allocates or frees device memory.  The plan is a small host
 *    object owned by the library (see latent_moe_free).
 *  - All work is enqueued on the caller's HIP stream (hipStream_t passed as
 *    void*; NULL = the default stream).  No call synchronises the stream or
 *    copies device data to the host; results are valid once the stream reaches
 *    the enqueued work.
 *  - Return value: LMOE_OK, or an error code.  On LMOE_EINVAL and
 *    LMOE_EUNSUPPORTED nothing was enqueued.  LMOE_EHIP reports a HIP launch
 *    error (some earlier kernels of the call may have been enqueued).  A
 *    device-side fault surfaces at the caller's next synchronisation.
 *    latent_moe_last_error() gives a one-line reason for the last failure on
 *    the calling thread.
 *  - All element offsets are computed in 64 bits.
 */
#ifndef LATENT_MOE_H
#define LATENT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LMOE_OK = 0, LMOE_EINVAL = 1, LMOE_EUNSUPPORTED = 2, LMOE_EHIP = 3 };
/* Routed-expert weight formats (lmoe_forward_args.wfmt):
 *  LMOE_WFMT_BF16        bf16 weights.
 *  LMOE_WFMT_MXFP4       MXFP4 weights, "w4a8": the expert GEMMs' activations are
 *                        quantised to MXFP8 and multiplied on the block-scaled
 *                        fp8 x fp4 MFMA (the large-batch mode).
 *  LMOE_WFMT_MXFP4_W4A16 the same MXFP4 weights, "w4a16": activations stay bf16;
 *                        the weights are upcast to bf16 inside the K loop and
 *                        multiplied on bf16 MFMAs (TokenSpeed Day-0 post,
 *                        "TensorRT-LLM Stable LatentMoE" and "Gluon kernels on
 *                        AMD GPUs > Stable LatentMoE").  Decode-shaped batches
 *                        (T*k <= 32*E) run weight-streaming kernels; larger ones
 *                        the tiled expert GEMMs, which upcast the weights to
 *                        bf16 (on their way into LDS, or from LDS into the
 *                        MFMA operands when K is a multiple of 512) and need
 *                        l, I >= 256 (else LMOE_EUNSUPPORTED, nothing
 *                        enqueued). */
enum { LMOE_WFMT_BF16 = 0, LMOE_WFMT_MXFP4 = 1, LMOE_WFMT_MXFP4_W4A16 = 2 };
/* Storage of bf16 routed-expert weights (lmoe_forward_args.wlayout):
 *  LMOE_WLAYOUT_ROWS   row-major [E, N, K] (the layout every shape below names).
 *  LMOE_WLAYOUT_TILED  tile-packed by latent_moe_pack_weights: the same values
 *                      in 128-row x 64-column blocks, each 16 KB contiguous,
 *                      so the expert GEMMs stream contiguous blocks.  Only for
 *                      LMOE_WFMT_BF16 with l and I multiples of 128, at least
 *                      256; results equal the row-major layout's bit for bit. */
enum { LMOE_WLAYOUT_ROWS = 0, LMOE_WLAYOUT_TILED = 1 };

/* Limits of this library. */
#define LMOE_MAX_EXPERTS_LOGITS 1024 /* E in logits mode (router keeps E/64 logits per lane) */
#define LMOE_MAX_EXPERTS 4096        /* E in ids mode */
#define LMOE_MAX_TOPK 64             /* k (one lane per selected expert) */
#define LMOE_MAX_SHARED 4            /* S */

typedef struct latent_moe_plan latent_moe_plan; /* opaque, host memory */

/*
 * Routing: router top-k/softmax (TokenSpeed AgentX post, "Model architecture":
 * each token picks k of E routed experts) and the per-expert permutation a
 * grouped-GEMM MoE builds (TokenSpeed Day-0 post, "Gluon kernels on AMD GPUs >
 * Stable LatentMoE": route sorting and gather buffers).
 *
 * Logits mode (logits != NULL, ids_in == NULL): for each token t,
 *   topk_ids[t,0..k-1] = the k experts with the largest logits, listed in the
 *   order (logit descending, expert index ascending); IEEE comparison, so +0
 *   and -0 tie and the lower index wins; NaN ranks below every number.
 *   topk_w[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0)   (fp32).
 * Ids mode (logits == NULL, ids_in != NULL): the caller supplies the expert
 *   of every row and its combine weight (one expert-parallel rank's received
 *   rows: k must be 1); topk_ids/topk_w, if not NULL, receive copies.
 * Both modes then build the stable counting sort of the rows r = t*k + j by
 * expert:  offsets[e] = number of rows with expert < e (E+1 entries,
 * offsets[E] = T*k);  sorted_row[p] = r, the p-th row in (expert, r)
 * ascending order;  row_pos[r] = p, its inverse.
 *
 * Arguments (device pointers unless noted):
 *   T           tokens (rows in ids mode), 0 <= T, T*k < 2^31
 *   E, k        experts and experts per token: 1 <= k <= min(E, 64);
 *               E <= 1024 in logits mode, E <= 4096 in ids mode
 *   logits      fp32 [T,E] or NULL
 *   ids_in      int32 [T,k], values in [0,E), or NULL.  The values are not
 *               checked: an id outside [0,E) is a caller error that the
 *               device code does not report (it is clamped to the nearest
 *               expert, 0 or E-1, so no access leaves the buffers)
 *   weights_in  fp32 [T,k] (ids mode only)
 *   topk_ids    int32 [T,k] out (logits mode: required)
 *   topk_w      fp32 [T,k] out (logits mode: required)
 *   sorted_row  int32 [T*k] out
 *   row_pos     int32 [T*k] out
 *   offsets     int32 [E+1] out
 *   workspace   >= latent_moe_route_workspace_size(T,E,k) bytes; holds the
 *               grouped-GEMM tile tables that latent_moe_forward reads
 * On success *out_plan receives a new plan that borrows (does not copy) the
 * output and workspace pointers: they must stay valid and unmodified for
 * every latent_moe_forward that uses the plan.  T == 0 is valid: no pointer
 * is read or checked, nothing is enqueued, and forward with that plan only
 * validates its dimensions and does nothing.
 */
typedef struct {
  int64_t T;
  int32_t E, k;
  const float* logits;
  const int32_t* ids_in;
  const float* weights_in;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* sorted_row;
  int32_t* row_pos;
  int32_t* offsets;
  void* workspace;
  size_t workspace_bytes;
} lmoe_route_args;

int latent_moe_route(const lmoe_route_args* args, void* hip_stream, latent_moe_plan** out_plan);

/*
 * Forward: down-projection, routed SwiGLU experts on grouped MFMA GEMMs,
 * gather-weight-accumulate combine with optional RMSNorm, shared experts, and
 * the up-projection (the formulas at the top of this file), using the routing
 * in `plan`.
 *
 * Dimensions: d (hidden), l (latent), I (routed intermediate), Is (shared
 * intermediate) are multiples of 64 (l and I multiples of 128 with MXFP4
 * weights); l <= 4096; 0 <= S <= 4 shared experts; wfmt is one of the
 * LMOE_WFMT_* values.
 * Arguments (device pointers, bf16 unless noted):
 *   x        [T,d]          hidden states (rows mode: latent rows [T,l])
 *   w_in     [l,d]          latent down-projection; NULL selects rows mode
 *   w1, w3   [E,I,l]        routed gate / up projections
 *                           (either MXFP4 format: u8 [E,I,l/2], two e2m1 codes
 *                           per byte, even K index in the low nibble)
 *   w2       [E,l,I]        routed down projection (MXFP4: u8 [E,l,I/2])
 *   s1, s3   u8 [E,I,l/32]  e8m0 block scales (MXFP4 formats only, else NULL)
 *   s2       u8 [E,l,I/32]
 *   norm_w   [l]            routed-latent RMSNorm gain, or NULL for no norm
 *   norm_eps                RMSNorm epsilon
 *   w_out    [d,l]          latent up-projection; NULL iff w_in is NULL
 *   ws1, ws3 [S,Is,d]       shared experts' gate / up (NULL iff S == 0)
 *   ws2      [S,d,Is]       shared experts' down projection
 *   y        [T,d] out      layer output.  Rows mode (one expert-parallel
 *                           rank's share; plan from ids mode, k == 1, S == 0):
 *                           y [T,l] = w[r] * Y[r], rows in received order.
 *   workspace >= latent_moe_forward_workspace_size(...) bytes (intermediates
 *             z, hs, H, Y, rhat and, for w4a8, the MXFP8 activation copies)
 *   wlayout  LMOE_WLAYOUT_ROWS, or LMOE_WLAYOUT_TILED for bf16 w1, w3, w2
 *            packed by latent_moe_pack_weights (see LMOE_WLAYOUT_*); a shape
 *            the packed layout does not serve returns LMOE_EUNSUPPORTED
 * Inputs are read-only; y and the workspace are written.  x, the weights and
 * y must not overlap the workspace.
 */
typedef struct {
  int32_t d, l, I, S, Is;
  int32_t wfmt;
  float norm_eps;
  const void* x;
  const void* w_in;
  const void* w1;
  const void* w3;
  const void* w2;
  const uint8_t* s1;
  const uint8_t* s3;
  const uint8_t* s2;
  const void* norm_w;
  const void* w_out;
  const void* ws1;
  const void* ws3;
  const void* ws2;
  void* y;
  void* workspace;
  size_t workspace_bytes;
  int32_t wlayout; /* LMOE_WLAYOUT_*: how bf16 w1, w3, w2 are stored (0 = row-major) */
} lmoe_forward_args;

int latent_moe_forward(const latent_moe_plan* plan, const lmoe_forward_args* args, void* hip_stream);

/*
 * The whole layer in one call: routing and the forward as above.  Two ways
 * to get the routing:
 *  - with a router gate (w_router != NULL) the logits are computed from the
 *    latent (vLLM Kimi K3 post, section 1: the latent down-projection is
 *    inserted in front of the router):
 *      z      = x W_in^T               (bf16, as in latent_moe_forward)
 *      logits = z W_router^T           fp32 [T,E], one fp32 accumulation per
 *                                      entry, not rounded
 *    then routing of `logits` as latent_moe_route in logits mode;
 *  - without one (w_router == NULL) the route arguments give the logits or
 *    the ids, exactly as for latent_moe_route.  Since the routing then does
 *    not depend on x, at T <= 512 in logits mode the top-k runs in the same
 *    launch as the down-projection and the shared experts' gate/up.
 * The results equal latent_moe_route followed by latent_moe_forward.
 * Arguments:
 *   route     as for latent_moe_route; with w_router, logits == NULL and
 *             ids_in == NULL, and topk_ids, topk_w are required (E <= 1024)
 *   w_router  bf16 [E,l] router gate (device), or NULL
 *   logits    with w_router: fp32 [T,E] out (device), the computed logits;
 *             without: must be NULL
 *   fwd       as for latent_moe_forward; w_in must not be NULL (no rows mode)
 *   plan_io   in/out.  *plan_io == NULL: a new plan is returned in it (free it
 *             with latent_moe_free).  Otherwise it must be a plan from an
 *             earlier latent_moe_layer call: it is refilled in place (its stage
 *             events are kept) and no host memory is allocated.
 * Errors as for the other calls; on LMOE_EINVAL and LMOE_EUNSUPPORTED nothing
 * was enqueued and *plan_io is unchanged.  On LMOE_EHIP a plan allocated by
 * this call is freed and *plan_io is set to NULL (a reused plan stays the
 * caller's).  With stage events set, stage 2 (events[1] -> events[2]) also
 * covers the gate GEMM (if any), the top-k and the permutation; where the
 * top-k shares the down-projection's launch it falls in stage 1.
 */
int latent_moe_layer(const lmoe_route_args* route, const void* w_router, float* logits,
                     const lmoe_forward_args* fwd, void* hip_stream, latent_moe_plan** plan_io);

/*
 * The whole layer for decode-shaped batches, organised around outputs rather
 * than experts (TokenSpeed Day-0 post, "Gluon kernels on AMD GPUs > Stable
 * LatentMoE": no route sorting, row padding or gather buffers).  The router's
 * top-k and softmax run as in latent_moe_layer (logits given); then each
 * expert-GEMM workgroup owns output columns of one expert and finds that
 * expert's (token, slot) rows by scanning topk_ids itself.  No permutation or
 * tile table is built, H and Y are kept in (token, slot) order, and the
 * combine reads Y there.  Where latent_moe_layer runs its weight-streaming
 * kernels (T*k <= 32*E) the results are equal to its results bit for bit:
 * each row meets the same MFMAs in the same K order.
 * Arguments as for latent_moe_layer with the logits given (w_router NULL):
 *   route   logits != NULL, ids_in == NULL; topk_ids and topk_w receive the
 *           routing; sorted_row, row_pos, offsets and workspace are not used
 *   fwd     as for latent_moe_forward; the forward workspace holds z, hs,
 *           H and Y (rows r = t*k + j) and rhat (same size and layout offsets)
 * Limits (else LMOE_EUNSUPPORTED, nothing enqueued): T <= 512, T*k <= 8192;
 * bf16 experts with l and I multiples of 128, or MXFP4 w4a16 experts with
 * l = I = 256; E <= 1024.  No plan is created.
 */
int latent_moe_layer_os(const lmoe_route_args* route, const lmoe_forward_args* fwd, void* hip_stream);

/*
 * latent_moe_layer for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It computes
 * exactly what latent_moe_layer computes (the same kernels), except that
 *  - both workspaces come from a static device array of
 *    LMOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 *    from the first call on that GPU until the process ends: route->workspace
 *    and fwd->workspace must be NULL and their sizes 0;
 *  - no plan is created or kept (no host allocation either); stage events do
 *    not apply.
 * Limit: latent_moe_route_workspace_size (rounded up to 256 bytes) plus
 * latent_moe_forward_workspace_size must not exceed the array, else
 * LMOE_EUNSUPPORTED and nothing is enqueued (64 MiB holds the decode shape,
 * 256 tokens x top-16 of 896 at latent 256, about 14 times over; a prefill
 * batch does not fit).
 * Every call on one GPU uses that GPU's one array: calls that overlap on the
 * same GPU (other streams, other host threads) race on it and must be
 * serialised by the caller.  The array keeps the last call's intermediates
 * (latent_moe_forward_workspace_layout at offset
 * round_up(latent_moe_route_workspace_size, 256)); no part of it needs to
 * start at zero.  The work runs on the device of hip_stream (the current
 * device for NULL).  Other arguments and errors as for latent_moe_layer.
 */
#define LMOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int latent_moe_layer_noalloc(const lmoe_route_args* route, const void* w_router, float* logits,
                             const lmoe_forward_args* fwd, void* hip_stream);

/*
 * Packs one bf16 routed-expert weight matrix [E, N, K] (w1 or w3: N = I,
 * K = l; w2: N = l, K = I) into the tile-packed layout LMOE_WLAYOUT_TILED:
 * element (e, n, k) moves to
 *   (((e * N/128 + n/128) * K/64 + k/64) * 128 + n%128) * 64 + k%64,
 * so that the 64 K columns of 128 consecutive rows of one expert are one
 * contiguous 16 KB block.  A load-time step (the expert GEMMs read each such
 * block whole in one pipeline stage); the values are copied unchanged.
 *   src, dst  device, bf16, E*N*K elements each, 16-byte aligned, not
 *             overlapping; dst is written, src only read
 *   N         a multiple of 128;  K a multiple of 64;  E >= 1
 * Enqueued on hip_stream; LMOE_EINVAL on invalid arguments (nothing enqueued).
 */
int latent_moe_pack_weights(const void* src, void* dst, int32_t E, int32_t N, int32_t K, void* hip_stream);

/* Releases a plan (host memory only; NULL is a no-op).  Device buffers the
 * plan borrowed remain the caller's. */
void latent_moe_free(latent_moe_plan* plan);

/* Optional stage timing (profiling aid, no effect on results).  With n ==
 * LMOE_N_STAGE_EVENTS caller-created hipEvent_t handles (passed as void*),
 * every later latent_moe_forward on this plan records events[0] before its
 * first kernel and events[i] after stage i: 1 down-projection, 2 shared
 * experts' gate/up (and, with MXFP4 experts, the MXFP8 quantisation of the
 * FC1 input where the down-projection's kernel does not write it in its
 * epilogue: rows mode and small T), 3 expert FC1, 4 expert FC2, 5 combine (+ RMSNorm),
 * 6 up-projection (stages a call does not run, or runs fused into the
 * previous stage's kernel, are recorded back to back).  events[2] and
 * events[3] are recorded by the FC1 launch itself (hipExtLaunchKernel) at
 * that kernel's start and end, so stage 3 is the FC1 kernel's own duration.
 * events == NULL (or n == 0) turns recording off.  The events are borrowed:
 * they must outlive their use.  Returns LMOE_EINVAL for a NULL plan or
 * another n. */
#define LMOE_N_STAGE_EVENTS 7
int latent_moe_plan_set_stage_events(latent_moe_plan* plan, void* const* events, int n);

/* Workspace sizes in bytes (0 on invalid dimensions).  rows_mode != 0 sizes
 * for an ids-mode plan with no projections. */
size_t latent_moe_route_workspace_size(int64_t T, int32_t E, int32_t k);
size_t latent_moe_forward_workspace_size(int64_t T, int32_t E, int32_t k, int32_t d, int32_t l,
                                         int32_t I, int32_t S, int32_t Is, int32_t wfmt,
                                         int32_t rows_mode);

/*
 * Where latent_moe_forward (and latent_moe_layer) keep the layer's
 * intermediates inside the forward workspace, for inspection and testing.
 * Every field is a byte offset from the workspace pointer; a field whose bit
 * is clear in `written` names storage that a forward with these dimensions
 * does not write.  The contents are valid once the stream has reached the end
 * of the call, until the workspace is used again.  Rows of H, Y, hq and hsc
 * are in permuted order: row p holds routed row sorted_row[p] = t*k + j.
 *   z    bf16 [T,l]      latent (not in rows mode)            LMOE_WS_Z
 *   hs   bf16 [T,S*Is]   shared experts' SwiGLU output         LMOE_WS_HS
 *   H    bf16 [T*k,I]    routed SwiGLU output (bf16 and w4a16 experts,
 *                        except the one-launch w4a16 expert MLP at
 *                        l = I = 256, which keeps H on chip)   LMOE_WS_H
 *   Y    bf16 [T*k,l]    routed expert output                  LMOE_WS_Y
 *   rhat bf16 [T,l]      combined routed latent after the RMSNorm
 *                        (not in rows mode)                    LMOE_WS_RHAT
 *   zq, zs  u8 [T,l], [T,l/32]    w4a8: MXFP8 codes and e8m0 scales of
 *                        FC1's input (z; rows mode: x)         LMOE_WS_ZQ
 *   hq, hsc u8 [T*k,I], [T*k,I/32] w4a8: MXFP8 codes and scales of H, which
 *                        FC1 writes in place of the bf16 H     LMOE_WS_HQ
 * Returns LMOE_OK, or LMOE_EINVAL for invalid dimensions or a NULL `out`
 * (then *out is unchanged).  Host only; nothing is enqueued.
 */
enum { LMOE_WS_Z = 1, LMOE_WS_HS = 2, LMOE_WS_H = 4, LMOE_WS_Y = 8, LMOE_WS_RHAT = 16, LMOE_WS_ZQ = 32,
       LMOE_WS_HQ = 64 };
typedef struct {
  size_t z, hs, H, Y, rhat, zq, zs, hq, hsc;
  size_t total; /* == latent_moe_forward_workspace_size(...) */
  uint32_t written; /* LMOE_WS_* bits */
} lmoe_forward_layout;

int latent_moe_forward_workspace_layout(int64_t T, int32_t E, int32_t k, int32_t d, int32_t l, int32_t I,
                                        int32_t S, int32_t Is, int32_t wfmt, int32_t rows_mode,
                                        lmoe_forward_layout* out);

/* One-line reason for the last non-OK status returned on this thread. */
const char* latent_moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LATENT_MOE_H */
