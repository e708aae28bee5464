/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE routing library:
 * token-to-expert routing with equal-cost load-balancing statistics.
 *
 * Pages cited (address, subject, section):
 *   [p1] mhpq.cn/news/998159 -- three layers of HPC load balancing; MoE
 *        part 4.2 (softmax router, argmax/top-k, f_i, P_i, aux loss), 4.4
 *        (top-k version: f_i over T*k assignments, histogram), 4.5 (capacity
 *        and token drop), 5.3/5.4 (f and P sum to one; max/mean load).
 *   [p2] codechina.net article 413310 -- equal-cost balancing in MoE
 *        training: 2.2 (L_aux = alpha*N*sum_i f_i*P_i; gradient only
 *        through P), 3.1 (histogram keeps zero-count experts), 3.2 (aux loss
 *        only in training), 4.2 (distribution ratio, entropy of the load).
 *   [p3] cnvsn.com/news/335486 -- load-balancing survey: 3.1 and 5.1
 *        (coefficient of variation, load-balance degree).
 *   [p1] 4.3 -- loss-free balancing: a per-expert scalar bias on the router
 *        logits, moved down for overloaded experts and up for idle ones.
 *   [p3] 4.1.2 -- EPLB: replicate heavily loaded experts, pack the replicas
 *        onto GPUs (balanced_packing).
 *   [p4] baidu-baige.github.io LoongForge blog on TAOT, section 2 Phase 1 --
 *        Sinkhorn-Knopp transport plan between overloaded and idle ranks.
 *
 * Conventions shared by every entry point:
 *   - Every array pointer is a DEVICE pointer to memory that the caller
 *     allocated and owns; the library never allocates, frees or keeps a
 *     pointer past the call.  Arrays are dense and row-major.
 *   - "stream" is a hipStream_t passed as an opaque pointer (NULL = the
 *     default stream).  All device work is enqueued asynchronously on it;
 *     no call synchronises the device.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     an error code nothing is launched and no output is touched.
 *   - T = tokens, E = experts, k = experts per token, m = n_micro
 *     microbatches of Tm = T/m tokens; each microbatch is routed on its own.
 *   - Ties between equal logits go to the lower expert index; -0.0 and +0.0
 *     are equal.  Results are deterministic: no floating-point atomics.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ROUTE_MAX_E 1024
#define MOE_ROUTE_MAX_K 32

/* Return codes. */
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1) /* NULL required pointer, bad shape or value */
#define MOE_ERR_UNSUPPORTED (-2) /* E, k or gate shape beyond the limits      */
#define MOE_ERR_WORKSPACE   (-3) /* workspace NULL or smaller than required   */
#define MOE_ERR_HIP         (-4) /* a HIP launch or runtime call failed       */
#define MOE_ERR_SCRATCH     (-5) /* moe_route_noalloc: the call needs more
                                    than MOE_ROUTE_SCRATCH_BYTES of scratch   */

/* moe_route_params.flags */
#define MOE_RENORM_TOPK    1u /* rescale the k gate weights to sum to 1     */
#define MOE_SAVE_ROW_STATS 2u /* write per-token softmax (max, sum)         */
#define MOE_WRITE_INV_PERM 4u /* write inv_perm                             */
#define MOE_SELECT_BIAS    8u /* moe_route's select_bias [E] steers the choice */
#define MOE_P_MASKED      16u /* P_e from each token's picks only, over Tm*k
                                 ([p1] 4.4's top-k code); default: the mean
                                 softmax over all tokens ([p1] 4.2)          */
#define MOE_MULTI_KERNEL  32u /* route the small microbatches moe_route
                                 takes in one launch (see there) with the
                                 multi-kernel path, as larger ones
                                 (integer outputs identical, floating-point
                                 ones up to summation order; for comparison) */

/* Bits of the optional status word (set for the whole call). */
#define MOE_STATUS_NONFINITE 1 /* a row had a NaN/+inf logit, or only -inf;
                                  outputs for such rows are unspecified     */
#define MOE_STATUS_INTERNAL  2 /* an internal bound check tripped          */

typedef struct {
    int32_t  T, E, k, n_micro; /* 1 <= k <= E <= MOE_ROUTE_MAX_E, k <= MOE_ROUTE_MAX_K,
                                  T % n_micro == 0, T*k < 2^31 */
    int32_t  d;                /* 0: logits are given; > 0: gate path, logits = X[T,d].Wg[d,E] */
    int32_t  capacity;         /* >= 0: per-microbatch capacity C; -1: from capacity_factor */
    double   capacity_factor;  /* used when capacity < 0; <= 0 means no limit (see
                                  moe_route_capacity for how it is rounded) */
    float    alpha;            /* aux-loss weight; 0 is legal (aux = 0, gradient = 0) */
    uint32_t flags;            /* MOE_* flags above */
} moe_route_params;

/*
 * Outputs of moe_route.  Arrays not marked "nullable" are required.
 *   topk_idx [T,k] int32   experts of token t, best first ([p1] 4.2, 4.4)
 *   topk_w   [T,k] fp32    gate weights: softmax probability of the pick,
 *                          or that divided by the sum over the k picks
 *                          (MOE_RENORM_TOPK)
 *   logits   [T,E] fp32    gate path only: the X.Wg logits are written here
 *                          (required when d > 0, ignored otherwise)
 *   row_stats[T,2] fp32    nullable; (max, sum of exp(l - max)) per token,
 *                          written when MOE_SAVE_ROW_STATS is set
 *   counts   [m,E] int32   assignments per expert before capacity
 *                          ([p1] 4.4, [p2] 3.1 -- zero-count experts kept)
 *   offsets  [m,E+1] int32 exclusive prefix sum of counts (segment-local)
 *   perm     [T*k] int32   expert-sorted dispatch order: the segment
 *                          [mb*Tm*k, (mb+1)*Tm*k) lists the flat indices
 *                          t*k+j of microbatch mb grouped by expert, experts
 *                          ascending, (t, j) ascending inside an expert
 *   inv_perm [T*k] int32   nullable; position in perm of assignment t*k+j,
 *                          written when MOE_WRITE_INV_PERM is set
 *   dropped  [T*k] uint8   1 when the assignment is the (C+1)-th or later of
 *                          its expert in its microbatch ([p1] 4.5)
 *   f, P     [m,E] fp32    nullable; f_e = counts/(Tm*k); P_e = mean over
 *                          the microbatch's tokens of softmax_e ([p1] 4.2),
 *                          or with MOE_P_MASKED the sum of softmax_e over the
 *                          tokens that picked e, divided by Tm*k ([p1] 4.4)
 *   aux_loss [m] fp32      alpha * E * sum_e f_e * P_e ([p2] 2.2)
 *   cv       [m] fp32      population std / mean of counts ([p3] 3.1)
 *   max_over_mean [m] fp32 max(counts) / mean ([p1] 5.4)
 *   extra_stats [m,8] fp32 nullable; min/mean, balance degree
 *                          1-(max-mean)/mean ([p3] 5.1), entropy of f (nats,
 *                          [p2] 4.2), kept, dropped, C (-1 = unlimited),
 *                          max f, min f ([p2] 4.2)
 *   status   [1] int32     nullable; MOE_STATUS_* bits of this call
 *   row_pass_events        nullable pair of hipEvent_t handles created by the
 *                          caller; when both are set the row-pass kernel (on
 *                          the one-launch path, that kernel) is launched
 *                          with them as its start and stop events
 *                          (hipExtLaunchKernel: the runtime stamps them from
 *                          that kernel's own dispatch, as a kernel trace
 *                          does; hipEventElapsedTime then gives its time)
 */
typedef struct {
    int32_t *topk_idx;
    float   *topk_w;
    float   *logits;
    float   *row_stats;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int32_t *inv_perm;
    uint8_t *dropped;
    float   *f;
    float   *P;
    float   *aux_loss;
    float   *cv;
    float   *max_over_mean;
    float   *extra_stats;
    int32_t *status;
    void    *row_pass_events[2];
} moe_route_out;

/*
 * Bytes of device workspace moe_route needs for these parameters (written to
 * *bytes).  The workspace holds per-block partial histograms and probability
 * sums; it needs no initialisation and its contents are scratch.
 */
int moe_route_workspace_size(const moe_route_params *p, size_t *bytes);

/*
 * Per-microbatch capacity C for these parameters (host only, no device
 * work).  [p1] 4.5 sets the capacity to the per-expert share of the batch,
 * rounded up, times the capacity factor (1024 tokens, 8 experts, 1.25 ->
 * 160); the k picks of a token count as k assignments, and a fractional
 * product is rounded up:  C = ceil(cf * n),  n = ceil(Tm*k/E).
 * The factor is the decimal the caller means (1.1, 1.2, ...), which a
 * double holds only to within half an ulp, so a product within 2^-50
 * (relative) of an integer is that integer: 1.1 * 50 gives 55 although the
 * double product is 55.000000000000007.  Exact for factors with at most
 * five decimal places.  -1 when unlimited (cf <= 0); the explicit capacity
 * field wins when >= 0; results above INT32_MAX are clamped to it.
 */
int moe_route_capacity(const moe_route_params *p, int32_t *capacity);

/*
 * Forward routing ([p1] 4.2-4.5, [p2] 2.2, [p3] 3.1/5.1).
 * logits [T,E] fp32 when p->d == 0 (X, Wg ignored); when p->d > 0, X [T,d]
 * and Wg [d,E] are bf16 bit patterns (uint16) and out->logits receives
 * X.Wg accumulated in fp32 (logits ignored).
 * select_bias [E] fp32: required when MOE_SELECT_BIAS is set, ignored
 * otherwise.  [p1] 4.3: the per-expert bias b_e is added to the logits to
 * steer the expert choice; here it enters the choice only -- experts are
 * ranked by the fp32 sum l + b_e (ties to the lower expert) while the gate
 * weights, P and the aux loss use the unbiased softmax.
 * Enqueues the whole forward on stream: the gate GEMM (gate path), then one
 * launch when E is 1, 2, 4 or 8, k*E <= 16, a microbatch holds at most
 * 32768 logits and there are at most 65535 microbatches (unless
 * MOE_MULTI_KERNEL), else a row pass, a block combine (skipped when the
 * scatter can sum the row blocks' partials itself) and the dispatch scatter.  workspace: device buffer of at
 * least moe_route_workspace_size() bytes, used only during the call's
 * kernels (calls sharing one workspace must be ordered on one stream).
 */
int moe_route(const moe_route_params *p, const float *logits, const uint16_t *X,
              const uint16_t *Wg, const float *select_bias, const moe_route_out *out,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_route for callers that cannot allocate device memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * same forward, with the workspace taken from a static device array of
 * MOE_ROUTE_SCRATCH_BYTES that the library holds on every GPU it runs on
 * (from the first call there until the process ends).  The caller still
 * passes the inputs and outputs, exactly as for moe_route; the call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * The scratch belongs to the device current on the calling thread, which
 * must be the device of stream.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (other streams, other threads)
 * race and must be ordered by the caller.  Nothing in the scratch needs to
 * start at zero; it holds the last call's partials.
 * Returns MOE_ERR_SCRATCH (nothing launched) when the shape needs more
 * workspace than MOE_ROUTE_SCRATCH_BYTES (moe_route_workspace_size tells);
 * otherwise the same codes as moe_route.
 */
#define MOE_ROUTE_SCRATCH_BYTES (32u * 1024u * 1024u)
int moe_route_noalloc(const moe_route_params *p, const float *logits, const uint16_t *X,
                      const uint16_t *Wg, const float *select_bias, const moe_route_out *out,
                      void *stream);

/*
 * One update of the selection bias after a forward ([p1] 4.3: an overloaded
 * expert's bias is pushed down, an idle expert's up, with no loss term).
 * The page fixes no step form; this is a fixed step against the sign of the
 * load error, in fp32:
 *   load_e = sum over microbatches of counts[mb][e];
 *   bias[e] -= gamma if load_e * E > T * k;  bias[e] += gamma if
 *   load_e * E < T * k;  unchanged if equal (exact integer comparison).
 * counts [m,E] int32: the forward's counts; bias [E] fp32: updated in
 * place.  Uses p->T, E, k, n_micro only.  gamma must be finite and >= 0.
 */
int moe_route_bias_update(const moe_route_params *p, const int32_t *counts, float gamma,
                          float *bias, void *stream);

/*
 * One loss-free balancing step ([p1] 4.3) in one call: moe_route with the
 * selection bias (p->flags must include MOE_SELECT_BIAS), then the bias step
 * of moe_route_bias_update from this call's counts, applied to select_bias in
 * place (read by the routing first, written after it).  The same results as
 * the two calls in sequence; with one microbatch on the multi-kernel path the
 * step is taken inside the dispatch scatter, which saves a launch.  gamma
 * must be finite and >= 0.  Other arguments, workspace and return codes as
 * for moe_route.
 */
int moe_route_with_bias_update(const moe_route_params *p, const float *logits, const uint16_t *X,
                               const uint16_t *Wg, float *select_bias, float gamma,
                               const moe_route_out *out, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Gradient with respect to the logits of
 *   L = sum_mb g_mb * aux_mb + sum_{t,j} d_topk_w[t,j] * topk_w[t,j]
 * with the forward's selection and counts held fixed ([p1] 4.2, [p2] 2.2:
 * f and the choice carry no gradient, the probabilities do):
 *   aux, all-token P:  dlogits[t,j] = g alpha E / Tm * p_j (f_j - sum_i f_i p_i)
 *   aux, MOE_P_MASKED ([p1] 4.4):  g alpha E / (Tm k) * p_j (f_j m_j -
 *                      sum_i f_i m_i p_i), m_i = 1 for t's picks
 *   gate weights:      the softmax Jacobian applied to d_topk_w; with
 *                      MOE_RENORM_TOPK through the renormalisation too
 *                      (then only the picked logits receive a gradient).
 * logits [T,E] fp32 (for the gate path: the logits moe_route wrote);
 * row_stats [T,2] nullable (the forward's MOE_SAVE_ROW_STATS output; NULL
 * recomputes them); counts [m,E] the forward's counts; d_aux [m] nullable
 * upstream gradient of each microbatch's aux loss (NULL = 1); topk_idx
 * [T,k] the forward's picks, required with MOE_P_MASKED or d_topk_w,
 * otherwise ignored; d_topk_w [T,k] nullable upstream gradient of the gate
 * weights (NULL = no weight term); dlogits [T,E] fp32 output.
 * Flags used: MOE_P_MASKED, MOE_RENORM_TOPK; capacity fields are ignored.
 */
int moe_route_backward(const moe_route_params *p, const float *logits,
                       const float *row_stats, const int32_t *counts,
                       const float *d_aux, const int32_t *topk_idx,
                       const float *d_topk_w, float *dlogits, void *stream);

/*
 * Backward of the gate GEMM logits = X.Wg (the gate network of [p2] 1.2):
 *   dX  = dlogits . Wg^T   [T,d] bf16 (fp32 accumulation, rounded to
 *                          nearest even), nullable
 *   dWg = X^T . dlogits    [d,E] fp32, nullable (at least one of the two)
 * Uses p->T, d (> 0) and E (same limits as the gate forward: d % 8 == 0,
 * E <= 64).  X [T,d] and Wg [d,E] are bf16 bit patterns; X and dX must be
 * 16-byte aligned.  dlogits [T,E] fp32 is the gradient with respect to the
 * logits (moe_route_backward's output).  workspace (for dWg only): at least
 * moe_gate_backward_workspace_size() bytes, 256-byte aligned; scratch.
 * Deterministic (fixed-order reductions, no atomics).
 */
int moe_gate_backward_workspace_size(const moe_route_params *p, size_t *bytes);
int moe_gate_backward(const moe_route_params *p, const uint16_t *X, const uint16_t *Wg,
                      const float *dlogits, uint16_t *dX, float *dWg, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * EPLB placement over expert loads ([p3] 4.1.2, global strategy), one
 * workgroup:
 *   replicate_experts: every expert starts with one replica; while fewer
 *   than num_phys replicas exist, the expert with the largest load per
 *   replica weight[e] / logcnt[e] gets another.  Physical replica i < E is
 *   expert i; replica E + r is the r-th copy made.
 *   balanced_packing: the replicas, each weighted weight / logcnt of its
 *   expert, are placed heaviest first into the lightest pack (GPU) that
 *   holds fewer than num_phys / num_packs replicas.
 * Per-replica loads compare exactly; ties go to the lower expert, replica
 * and pack index.  weight [E] int32 >= 0 (e.g. a row of moe_route's
 * counts; negative values count as 0).  Outputs: phy2log [num_phys]
 * (expert of each replica), phy_rank [num_phys] (replica number within its
 * expert), logcnt [E] (replicas per expert), pack [num_phys] and slot
 * [num_phys] (the replica's pack and position in it), pack_load
 * [num_packs] fp64 (8-byte aligned).
 * Limits: 1 <= E <= MOE_ROUTE_MAX_E, E <= num_phys <= MOE_EPLB_MAX_PHYS,
 * 1 <= num_packs <= MOE_EPLB_MAX_PACKS, num_phys % num_packs == 0.
 */
#define MOE_EPLB_MAX_PHYS  4096
#define MOE_EPLB_MAX_PACKS 1024
int moe_eplb_plan(int32_t E, int32_t num_phys, int32_t num_packs, const int32_t *weight,
                  int32_t *phy2log, int32_t *phy_rank, int32_t *logcnt, int32_t *pack,
                  int32_t *slot, double *pack_load, void *stream);

/*
 * Sinkhorn-Knopp flow plan ([p4] TAOT section 2, Phase 1), one workgroup:
 * supply a [R] (each rank's overload), demand b [R] (idle capacity; the
 * totals should be equal), cost [R,R] row-major (topology cost between
 * ranks), eps > 0 the entropy regularisation.  Gibbs kernel
 * K = exp(-cost / eps); from u = v = 1, each of the iters rounds sets
 *   u_i = a_i / max(sum_j K_ij v_j, 1e-300), then v_j = b_j / max(sum_i K_ij u_i, 1e-300);
 * outputs u [R], v [R] and the plan T [R,R] = diag(u) K diag(v).  All fp64,
 * 8-byte aligned.  Limits: 1 <= R <= MOE_SINKHORN_MAX_R,
 * 0 <= iters <= MOE_SINKHORN_MAX_ITERS.
 */
#define MOE_SINKHORN_MAX_R     64
#define MOE_SINKHORN_MAX_ITERS 100000
int moe_sinkhorn_plan(int32_t R, const double *supply, const double *demand, const double *cost,
                      double eps, int32_t iters, double *u, double *v, double *T, void *stream);

/* Static message for a return code. */
const char *moe_route_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
