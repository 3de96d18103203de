/*
 * lmoe.h - C ABI of the Stable LatentMoE forward pass and the Quantile
 * Balancing estimator on one AMD Instinct MI355X (gfx950).
 *
 * Sources (three web pages on the Kimi K3 architecture):
 *   [DD] "Kimi K3 Architecture Deep Dive": §1 SiTU-GLU, §2 Stable LatentMoE,
 *        §3 Quantile Balancing.
 *   [IK] "Inside K3: How Stable Latent MoE and MLA Attention Are Designed":
 *        sections SiTU-GLU, RMSNorm insertion, Quantile Balancing (QB).
 *   [RB] LeiPhone report on Su Jianlin's K3 notes: "LatentMoE: paying for a
 *        bigger pool", "Keeping the numbers in range".
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) unless
 *     stated; matrices are row-major with the PyTorch [out, in] weight layout.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     memory and keeps no state between calls (beyond launch settings it
 *     looks up once per kernel and device, thread-safely), so calls on
 *     different streams, devices or host threads with different workspaces
 *     may run concurrently.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; no entry point synchronises with the host.
 *   - Arguments are validated before anything is enqueued; on a validation
 *     error nothing is launched and a negative lmoe_status is returned.  A
 *     failed launch returns LMOE_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Pointers must be 16-byte aligned (LMOE_ERR_ALIGN otherwise).
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMOE_OK = 0,
  LMOE_ERR_NULL = -1,      /* a required pointer is NULL                       */
  LMOE_ERR_SHAPE = -2,     /* dims violate the layer's or the kernels' rules   */
  LMOE_ERR_DTYPE = -3,     /* unknown work dtype                               */
  LMOE_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned                 */
  LMOE_ERR_WORKSPACE = -5, /* workspace smaller than lmoe_workspace_size()     */
  LMOE_ERR_HIP = -6,       /* a HIP launch or runtime call failed              */
  LMOE_ERR_VALUE = -7,     /* a scalar argument is out of range                */
  LMOE_ERR_SCRATCH = -8    /* lmoe_forward_static: the call needs more scratch
                              than LMOE_STATIC_SCRATCH_BYTES                     */
} lmoe_status;

/* Work dtype: the storage type of x, the weights, and the stored activations
 * z, a, v, y.  Accumulation, router scores, routing weights, the aggregated
 * latent and the norm statistics are always fp32.  The k routed contributions
 * g_ie * (a W3_e^T) of a token are staged in the workspace before their fp32
 * sum: in fp16 when the work dtype is bf16 and both caps are finite (an
 * element beyond +-65504 becomes +-inf and so shows in y; the gated hidden a is
 * bounded by beta1 * beta2, so this needs a W3 row whose absolute values sum
 * past 65504 / (beta1 * beta2)), in fp32 when either cap is +inf (the hidden is
 * then unbounded) and when the work dtype is fp32. */
typedef enum { LMOE_F32 = 0, LMOE_BF16 = 1 } lmoe_dtype;

/* Layer dimensions ([DD] §2: d -> d/2 -> D -> d/2 -> d, k of n routed experts;
 * [RB] "LatentMoE: paying for a bigger pool": hidden 7168, latent 3584,
 * 16 of 896 routed experts, two always-on shared experts).
 *   T         tokens (>= 0; T == 0 is a successful no-op)
 *   d         model width; multiple of 128 (so that L is a multiple of 64)
 *   L         latent width; must equal d / 2
 *   n         routed experts, 1..1024
 *   k         experts chosen per token, 1..min(n, 64)
 *   n_shared  shared experts, 0..8
 *   D         expert hidden width; multiple of 64
 * Also d <= 65536, L <= 8192, D <= 65536 and T * (k + n_shared) < 2^31; and,
 * since the large GEMMs address each operand through 32-bit byte offsets,
 * every activation and weight matrix they read must span less than 4 GiB at
 * the work dtype: T*d, T*L, T*(k + n_shared)*D, L*d, n*L and 2*D*L elements
 * (lmoe_backward adds d, L and n rounded up to 64 times T rounded up to 64,
 * and L and 2*D times the padded expert-row count, about T*(k + n_shared) +
 * 128*(n + n_shared)).  Dims outside these rules give LMOE_ERR_SHAPE (and a
 * workspace size of 0).                                                      */
typedef struct {
  int64_t T, d, L, n, k, n_shared, D;
} lmoe_dims;

/* Expert caps ("Kimi K3 Architecture Deep Dive" §1 and "Inside K3", section
 * SiTU-GLU, contrast the tanh softcap with the hard clip it replaces):
 *   LMOE_GATE_TANH  softcap(x; beta) = beta tanh(x / beta): SiTU-GLU, the layer
 *                   as the pages define it
 *   LMOE_GATE_CLIP  clamp(x; beta) = min(max(x, -beta), beta) in both branches,
 *                   same beta1 and beta2: the hard-clip ablation
 * Any other value is rejected with LMOE_ERR_VALUE. */
typedef enum { LMOE_GATE_TANH = 0, LMOE_GATE_CLIP = 1 } lmoe_gate;

/* The norm before the up-projection ("Kimi K3 Architecture Deep Dive" §2 keeps
 * this one RMSNorm and no other):
 *   LMOE_NORM_RMS   v = rms_gain * u / sqrt(mean(u^2) + rms_eps): the layer as
 *                   the pages define it
 *   LMOE_NORM_NONE  v = u (rms_gain and rms_eps unused): the ablation
 *   LMOE_NORM_BOTH  LMOE_NORM_RMS plus the norm the pages leave out after the
 *                   down-projection: the stored z becomes
 *                   z / sqrt(mean(z^2) + rms_eps) (unit gain) before routing,
 *                   so the router and the experts both see it: the ablation
 * Any other value is rejected with LMOE_ERR_VALUE. */
typedef enum { LMOE_NORM_RMS = 0, LMOE_NORM_NONE = 1, LMOE_NORM_BOTH = 2 } lmoe_norm;

/* Weights (device pointers, work dtype unless noted).
 *   w_down [L, d]        down-projection, no bias ([DD] §2: pure linear map)
 *   w_router [n, L]      router; scores s = sigmoid(z w_router^T + o)
 *   router_bias [n] fp32 loss-free selection bias b: added to s for the top-k
 *                        choice only ([DD] §3; [RB] "Keeping the numbers in
 *                        range")
 *   router_logit_offset [n] fp32 or NULL: per-expert offset o added to the
 *                        logits before the sigmoid (a hook to make routing
 *                        skewed in synthetic workloads)
 *   w1, w2 [n, D, L]     SiTU gate branch / softcapped linear branch
 *   w3 [n, L, D]         expert output projection
 *   ws1, ws2 [n_shared, D, L], ws3 [n_shared, L, D]   shared experts (NULL iff
 *                        n_shared == 0); SiTU-GLU in the latent space, weight 1
 *   rms_gain [L]         gain of the single RMSNorm ([DD] §2: kept before the
 *                        up-projection only)
 *   w_up [d, L]          up-projection
 *   beta1, beta2         SiTU and softcap caps ([DD] §1: 4 and 25), in
 *                        (0, +inf]; +inf is the uncapped limit (softcap
 *                        becomes the identity, SiTU becomes SiLU), so both at
 *                        +inf give the SwiGLU expert the caps replace
 *   rms_eps              RMSNorm epsilon (>= 0; 1e-6 by default)
 *   gate                 lmoe_gate: how both expert branches are capped
 *   norm                 lmoe_norm: the norm before the up-projection          */
typedef struct {
  const void *w_down;
  const void *w_router;
  const float *router_bias;
  const float *router_logit_offset;
  const void *w1, *w2, *w3;
  const void *ws1, *ws2, *ws3;
  const void *rms_gain;
  const void *w_up;
  float beta1, beta2, rms_eps;
  int32_t gate;
  int32_t norm;
} lmoe_weights;

/* Bytes of device workspace lmoe_forward needs for these dims and dtype
 * (0 for invalid dims). */
size_t lmoe_workspace_size(const lmoe_dims *dims, int dtype);

/* Workspace regions that can be inspected after a forward (for tests and
 * debugging; contents are valid once the stream reaches the end of the call). */
typedef enum {
  LMOE_WS_Z = 0,         /* [T, L] work dtype: latent z = x w_down^T                    */
  LMOE_WS_COUNTS = 1,    /* [n] int32: tokens routed to each expert                      */
  LMOE_WS_OFFS = 2,      /* [n+1] int32: exclusive prefix sum of counts                  */
  LMOE_WS_ROW_TOKEN = 3, /* [T*(k+n_shared)] int32: token of each expert row.  Rows 0 ..
                                   T*k-1 are the dispatched (token, expert) pairs ordered
                                   by (expert, token); row T*k + s*T + t is token t of
                                   shared expert s                                        */
  LMOE_WS_ROW_SLOT = 4,  /* [T*k] int32: dispatched row of (token t, slot r) at t*k+r      */
  LMOE_WS_HIDDEN = 5,    /* [T*(k+n_shared), D] work dtype: gated hidden a of each row     */
  LMOE_WS_ROWS = 6,      /* [T*(k+n_shared), L] staged expert outputs: routed rows scaled
                                   by g, shared rows by 1; fp16 for bf16 work dtype with
                                   both caps finite, else fp32 (the region is sized for
                                   fp32 either way)                                       */
  LMOE_WS_V = 7          /* [T, L] work dtype: v = RMSNorm(u)                             */
} lmoe_ws_region;

/* Byte offset of a region inside the workspace (-1 for an invalid request). */
int64_t lmoe_workspace_offset(const lmoe_dims *dims, int dtype, int region);

/* Forward pass of one Stable LatentMoE layer ([DD] §1-§3; [IK]; [RB]):
 *   z = x w_down^T                      (stored in the work dtype)
 *   s = sigmoid(z w_router^T + o)       (fp32)
 *   K_i = top-k of s_i + b, ties -> lower expert index, ordered by decreasing
 *         biased score
 *   g_ie = s_ie / sum_{e' in K_i} s_ie'
 *   per routed expert e and each row routed to it:
 *     a = SiTU(z W1_e^T; beta1) * softcap(z W2_e^T; beta2)   (work dtype)
 *     u_i += g_ie * (a W3_e^T)
 *   u_i += sum_j W3s_j (SiTU(W1s_j z_i; beta1) * softcap(W2s_j z_i; beta2))
 *   v = rms_gain * u / sqrt(mean(u^2) + rms_eps)  (work dtype)
 *   y = v w_up^T                        (work dtype)
 * where softcap(x; b) = b tanh(x / b) and SiTU(x; b) = softcap(x; b) sigmoid(x);
 * with w->gate == LMOE_GATE_CLIP every softcap above is clamp(x; b) instead,
 * with w->norm == LMOE_NORM_NONE, v = u (work dtype), and with LMOE_NORM_BOTH
 * z is normed in place first (see lmoe_norm).
 * Arguments:
 *   x [T, d]      input tokens, work dtype
 *   y [T, d]      output, work dtype (may not alias x)
 *   topk_idx [T, k] int32 out, or NULL
 *   topk_w [T, k] fp32 out (g), or NULL
 *   scores [T, n] fp32 out (unbiased sigmoid scores, the input of
 *                 lmoe_qb_update), or NULL
 *   workspace     device buffer of at least lmoe_workspace_size() bytes,
 *                 16-byte aligned; its contents need no initialisation.
 * Routing is dropless: no capacity limit, every chosen (token, expert) pair is
 * computed.  NaN in x propagates to y. */
int lmoe_forward(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, void *y,
                 int32_t *topk_idx, float *topk_w, float *scores, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Bytes of the library's own device scratch used by lmoe_forward_static, one
 * copy per device (64 MiB: the workspace of decode-sized calls, e.g. up to
 * about 100 tokens at d = 7168 with 896 experts choose 16). */
#define LMOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* lmoe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with the workspace taken from a static device
 * array the library holds (LMOE_STATIC_SCRATCH_BYTES per device, looked up on
 * the first call on each device).  The caller still passes x, y and the
 * optional outputs.  Calls whose lmoe_workspace_size() exceeds
 * LMOE_STATIC_SCRATCH_BYTES return LMOE_ERR_SCRATCH before anything is
 * launched; the other errors are lmoe_forward's.  No memory is allocated or
 * freed.  The scratch keeps the last call's contents; the forward needs none of
 * it initialised.  Every call on one device shares that device's scratch:
 * calls that may overlap on one device (different streams, host threads) race
 * and must be serialised by the caller. */
int lmoe_forward_static(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, void *y,
                        int32_t *topk_idx, float *topk_w, float *scores, void *stream);

/* Stages of lmoe_forward, in launch order (for lmoe_forward_timed). */
#define LMOE_N_STAGES 8
/*  0 down-projection GEMM             4 W1/W2 + SiTU-GLU of every expert row
 *  1 router GEMM + sigmoid              (routed and shared, one grouped GEMM)
 *  2 top-k + routing weights          5 W3 of every expert row, scaled (grouped)
 *  3 dispatch permutation (3 kernels) 6 combine + RMSNorm
 *                                     7 up-projection GEMM                      */

/* lmoe_forward with per-stage timing: events is an array of n_events ==
 * LMOE_N_STAGES + 1 hipEvent_t handles created by the caller; events[i] is
 * recorded on `stream` before stage i and events[LMOE_N_STAGES] after the last
 * one, so hipEventElapsedTime(events[i], events[i+1]) is stage i's duration.
 * An entry may be NULL: that boundary is not recorded (each record costs a few
 * microseconds of stream time, so a caller timing one stage passes two).
 * Computes exactly what lmoe_forward computes (same kernels, same results).
 * Errors: events NULL -> LMOE_ERR_NULL; n_events wrong -> LMOE_ERR_VALUE. */
int lmoe_forward_timed(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, void *y,
                       int32_t *topk_idx, float *topk_w, float *scores, void *workspace,
                       size_t workspace_bytes, void *const *events, int n_events, void *stream);

/* Quantile Balancing update ([DD] §3: scores in [0,1] -> B-bin histogram ->
 * histograms summed across devices -> quantile read; [IK] Quantile Balancing;
 * [RB] "Keeping the numbers in range": each expert's threshold is moved to
 * where it receives its target share).
 *   scores [T, n] fp32    unbiased router scores (as written by lmoe_forward);
 *                         0 <= T < 2^31, 1 <= n <= 2^20, 1 <= k <= n
 *   nbins                 B, 1..16384 (1000 by default on the pages)
 *   hist [n, nbins] int32 per-expert histogram, in/out.  With accumulate == 0 it
 *                         is overwritten by this batch's counts; with
 *                         accumulate == 1 the batch's counts are added (the
 *                         single-device form of the cross-device sum).
 *                         bin(s) = min(B-1, floor(fp32(s * B))) for s*B >= 1,
 *                         else 0 (negative scores and NaN go to bin 0).
 *   bias [n] fp32         written only if solve != 0:
 *                           N_e  = sum_j hist[e][j]
 *                           q_e  = read(hist[e], N_e * k / n)
 *                           tau  = read(sum_e hist[e], (sum_e N_e) * k / n)
 *                           bias[e] = fp32(tau - q_e)     (computed in fp64)
 *                         where read(h, c) = (j* + 1 - (c - G(j*+1)) / h[j*]) / B,
 *                         G(j) = sum_{j' >= j} h[j'], j* = max{j : G(j) >= c}.
 *                         Experts with an empty histogram keep their bias.
 *   workspace             device buffer of lmoe_qb_workspace_size(n, nbins) bytes
 *                         when T > 0 or solve != 0 (may be NULL otherwise): the
 *                         pooled histogram and the token runs' count slabs
 * T == 0 with accumulate == 0 clears the histogram.  Counts are int32: the
 * caller keeps every bin below 2^31 across accumulated batches. */
int lmoe_qb_update(const float *scores, int64_t T, int64_t n, int64_t k, int32_t nbins,
                   int32_t *hist, int accumulate, float *bias, int solve, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Bytes of device workspace lmoe_qb_update needs for n experts and nbins bins
 * (the pooled histogram, int64 [nbins], tau and a completion counter, n
 * doubles of per-expert reads, then up to 16 int32 [n, nbins] slabs of per-run
 * counts); 0 for an invalid n or nbins. */
size_t lmoe_qb_workspace_size(int64_t n, int32_t nbins);

/* Gradients of the layer (device pointers, work dtype, overwritten).  Shapes as
 * the weights they belong to; dws* NULL iff n_shared == 0. */
typedef struct {
  void *dx;          /* [T, d]        gradient of the input x                    */
  void *dw_down;     /* [L, d]                                                   */
  void *dw_router;   /* [n, L]                                                   */
  void *dw1, *dw2;   /* [n, D, L]                                                */
  void *dw3;         /* [n, L, D]                                                */
  void *dws1, *dws2; /* [n_shared, D, L]                                         */
  void *dws3;        /* [n_shared, L, D]                                         */
  void *dgamma;      /* [L]           gradient of rms_gain                       */
  void *dw_up;       /* [d, L]                                                   */
} lmoe_grads;

/* Bytes of device workspace lmoe_backward needs (0 for invalid dims or dtype,
 * or a latent width above 4096). */
size_t lmoe_backward_workspace_size(const lmoe_dims *dims, int dtype);

/* Backward pass of the layer ("Kimi K3 Architecture Deep Dive" §1: the capped
 * gate SiTU(x1) softcap(x2); §2: the norm before the up-projection, whose
 * weight gradient takes the normalised form g (h / |h|_RMS)^T): the gradients
 * of x and of every weight for the upstream gradient dy [T, d] of y.
 * Call after lmoe_forward on the same stream, with the same dims, weights,
 * dtype and x, passing that forward's topk_idx, topk_w and scores outputs (all
 * required) and its workspace, untouched since (it holds z, the routing, the
 * gated hidden, the staged expert rows and v).  Steps, with the forward's
 * notation, r the token's RMS and u_hat = u / r:
 *   dv = dy w_up;  dw_up = dy^T v;  dgamma = sum_i dv (.) u_hat
 *   du = (gamma (.) dv - u_hat mean(gamma (.) dv (.) u_hat)) / r   (LMOE_NORM_RMS;
 *        du = dv with LMOE_NORM_NONE)
 *   per expert row (token i, weight g; shared rows g = 1):
 *     da  = g (du_i W3_e);  dw3_e += (g du_i)^T a
 *     dp1 = da C(p2) SiTU'(p1),  dp2 = da SiTU(p1) C'(p2)  (p1, p2 recomputed
 *           from z; C the branch cap, C'(x) = 1 - tanh^2(x / beta), or 1 inside
 *           the clip's range and 0 outside)
 *     dz_i += dp1 W1_e + dp2 W2_e;  dw1_e += dp1^T z_i;  dw2_e += dp2^T z_i
 *   router, chosen experts only (the selection and the bias have no gradient):
 *     dg_j = du_i . o_j;  ds_j = (dg_j - sum_j' dg_j' g_j') / S;
 *     dl_j = ds_j s_j (1 - s_j);  dz += dl w_router;  dw_router = dl^T z
 *   dx = dz w_down;  dw_down = dz^T x
 * du, g du, da, dp1, dp2, dl, dz and the per-slot rows dz is summed from are
 * stored in the work dtype between steps; sums run in fp32.  Restrictions: LMOE_NORM_BOTH is not supported
 * (LMOE_ERR_VALUE); L <= 4096 (LMOE_ERR_SHAPE).  T == 0 writes zero weight
 * gradients.  workspace: lmoe_backward_workspace_size() bytes.
 * Ownership and errors: every buffer is the caller's (device pointers, 16-byte
 * aligned, LMOE_ERR_ALIGN otherwise); the gradients must not overlap each
 * other, the inputs or either workspace; the expert weights are read in their
 * stored layout.  All arguments are checked before anything is launched
 * (LMOE_ERR_NULL for a missing required pointer or, with shared experts, a
 * missing shared gradient; LMOE_ERR_SHAPE for shared gradients without shared
 * experts; LMOE_ERR_WORKSPACE when either workspace is too small); a launch
 * that fails returns LMOE_ERR_HIP.  The call does not synchronise with the
 * host; calls that share a workspace must not overlap. */
int lmoe_backward(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, const void *dy,
                  const int32_t *topk_idx, const float *topk_w, const float *scores, const void *fwd_workspace,
                  size_t fwd_workspace_bytes, const lmoe_grads *grads, void *workspace, size_t workspace_bytes,
                  void *stream);

/* Margin form of the Quantile Balancing update ("Kimi K3 Architecture Deep
 * Dive" §3; LeiPhone report "Keeping the numbers in range": the router scores
 * are read against each token's top-k threshold to estimate where each
 * expert's threshold must move to receive its target share).
 *   scores [T, n] fp32    unbiased router scores; 0 <= T < 2^31, 1 <= n <= 1024,
 *                         1 <= k <= n
 *   bias [n] fp32         in: the bias the margins are taken against (the one
 *                         the scores were routed with); out (solve != 0): the
 *                         updated bias
 *   hist [n, nbins] int32 in/out, overwritten (accumulate == 0) or added to
 * Per token i, with keys sel_ie = fp32(s_ie + b_e): tk_i / tk1_i = its k-th /
 * (k+1)-th largest key (tk1 = -inf when k == n).  The margin of (i, e) is
 *   m_ie = fp32(sel_ie - tk1_i) if sel_ie >= tk_i, else fp32(sel_ie - tk_i),
 * the bias shift at which e leaves or enters token i's top-k; it is binned as
 * the score rule of lmoe_qb_update applied to u = fp32(m + 1) * 0.5.  The
 * solve reads q_e = read(hist[e], N_e * k / n) (as lmoe_qb_update) and sets
 *   bias[e] = fp32(bias[e] - (2 q_e - 1))    (computed in fp64);
 * experts with an empty histogram keep their bias.  All operations are in a
 * fixed order, so the result is reproducible bit for bit.
 *   workspace             device buffer of lmoe_qb_margin_workspace_size(T, n,
 *                         nbins) bytes (the per-token thresholds, then the
 *                         token runs' count slabs); may be NULL when T == 0
 * T == 0 with accumulate == 0 clears the histogram. */
int lmoe_qb_margin_update(const float *scores, int64_t T, int64_t n, int64_t k, int32_t nbins, int32_t *hist,
                          int accumulate, float *bias, int solve, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Bytes of device workspace lmoe_qb_margin_update needs for T tokens, n experts
 * and nbins bins (0 for an invalid T, n or nbins). */
size_t lmoe_qb_margin_workspace_size(int64_t T, int64_t n, int32_t nbins);

/* The fixed-step bias update of K2's loss-free balancing that Quantile
 * Balancing replaces ("Kimi K3 Architecture Deep Dive" §3: SignSGD-style,
 * unstable at 896 experts; LeiPhone report "Keeping the numbers in range":
 * selection nudged up or down by a fixed step):
 *   load_e  = number of entries equal to e in topk_idx [T, k] (int32)
 *   bias[e] = fp32(bias[e] + step * sign(T k - load_e n))
 * i.e. a step up below the share T k / n, down above it, none at it.  The
 * pages give no step size: `step` is the caller's (finite).  Entries outside
 * [0, n) are not counted.  T == 0 is a no-op (topk_idx may then be NULL). */
int lmoe_bias_signsgd(const int32_t *topk_idx, int64_t T, int64_t n, int64_t k, float step, float *bias,
                      void *stream);

/* Static description of a status code. */
const char *lmoe_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LMOE_H */
