/*
 * moe_oracle.c -- plain, slow CPU oracle for MoE token routing with
 * equal-cost load-balancing statistics.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * Every step is the plain definition written out in double precision, in
 * the order the pages give it.  Pages cited (address, title, section):
 *   [p1] mhpq.cn/news/998159, on the three layers of HPC load balancing
 *        (LVS, NIC Teaming, MoE equal-cost balancing): section 4.2 (f_i,
 *        P_i, aux loss), 4.4 (top-k version, f_i denominator), 4.5
 *        (capacity), 5.3/5.4 (sanity sums, max/mean load).
 *   [p2] codechina.net article 413310, "equal-cost load balancing in MoE
 *        training: principles, code, tuning": section 2.2 (the aux loss and
 *        its value 1 under uniform routing), 3.1 (histogram keeps
 *        zero-count experts), 4.2 (distribution ratio, entropy).
 *   [p3] cnvsn.com/news/335486, survey of load balancing for large models:
 *        sections 3.1 and 5.1 (coefficient of variation, balance degree).
 *   [p3] section 4.1.2 (EPLB): replicate_experts copies the expert with the
 *        highest load per replica until the physical-expert count is reached;
 *        balanced_packing sorts items by weight (descending) and puts each
 *        into the lightest bin that is not full; worked example [9,7,5,3]
 *        into 2 bins of 2 -> loads 12 and 12.
 *   [p4] baidu-baige.github.io LoongForge blog on TAOT (topology-aware optimal
 *        transport for expert replicas), section 2 Phase 1: overload of each
 *        rank as supply, idle capacity as demand, a topology cost matrix, and
 *        the entropy-regularised plan T = diag(u) K diag(v) computed by
 *        alternating Sinkhorn-Knopp matrix-vector steps (about 50 rounds).
 *   [p1] section 4.3 also gives the loss-free variant: a per-expert scalar
 *        bias on the router logits, moved down for overloaded experts and up
 *        for idle ones (selection bias and its update, below).
 * Readings where the pages are silent are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double (exact: bf16 is the upper half of an fp32). */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

/*
 * Per-microbatch expert capacity.  [p1] 4.5 sets it to the tokens-per-
 * expert share of the batch, rounded up, times the capacity factor; its
 * worked example is 1024 tokens, 8 experts, factor 1.25 -> 160.
 * Reading for top-k (k assignments per token): the load to spread is Tm*k
 * assignments, and a fractional product with the factor is rounded up:
 *   C = ceil(cf * ceil(Tm*k / E)).
 * The factor is the decimal number the caller wrote ("1.1", "1.25",
 * "5e-1"), taken as text so that it is exact: cf = M * 10^-D with integer
 * M, and the product is formed and rounded up in integer arithmetic, so an
 * integral product stays integral (1.1 * 50 = 55).
 * cf <= 0 means "no limit" (returned as -1).  A non-negative override wins.
 * A capacity above 2^31 - 1 (more than any call's assignments) is returned
 * as 2^31 - 1.  Returns -2 when the text is not a decimal number.
 */
long long oracle_capacity(long long Tm, long long E, long long k, const char *cf_text,
                          long long capacity_override)
{
    const long long cap_max = 2147483647LL;
    if (capacity_override >= 0)
        return capacity_override;
    /* parse [+|-]digits[.digits][(e|E)[+|-]digits] into M and D */
    const char *c = cf_text;
    int neg = 0, digits = 0, frac = 0, seen_dot = 0;
    unsigned __int128 M = 0;
    if (*c == '+' || *c == '-')
        neg = (*c++ == '-');
    for (; *c; ++c) {
        if (*c == '.' && !seen_dot) {
            seen_dot = 1;
        } else if (*c >= '0' && *c <= '9') {
            if (M > (((unsigned __int128)1) << 100))
                return -2; /* more digits than any double's decimal form */
            M = M * 10 + (unsigned)(*c - '0');
            frac += seen_dot;
            ++digits;
        } else {
            break;
        }
    }
    long long ex = 0;
    if (*c == 'e' || *c == 'E') {
        ++c;
        int eneg = 0;
        if (*c == '+' || *c == '-')
            eneg = (*c++ == '-');
        if (!(*c >= '0' && *c <= '9'))
            return -2;
        for (; *c >= '0' && *c <= '9'; ++c)
            if (ex < 100000)
                ex = ex * 10 + (*c - '0');
        ex = eneg ? -ex : ex;
    }
    if (*c != '\0' || digits == 0)
        return -2;
    if (neg || M == 0)
        return -1;
    long long D = frac - ex; /* cf = M * 10^-D */
    long long per_expert = (Tm * k + E - 1) / E; /* ceil(Tm*k/E) */
    unsigned __int128 num = M * (unsigned __int128)per_expert;
    unsigned __int128 cap;
    if (D <= 0) {
        cap = num;
        for (long long i = 0; i < -D && cap <= (unsigned __int128)cap_max; ++i)
            cap *= 10;
    } else if (D > 38) {
        cap = (num > 0) ? 1 : 0; /* 0 < cf * n < 1 */
    } else {
        unsigned __int128 den = 1;
        for (long long i = 0; i < D; ++i)
            den *= 10;
        cap = (num + den - 1) / den;
    }
    return cap > (unsigned __int128)cap_max ? cap_max : (long long)cap;
}

/*
 * Gate GEMM: logits[t][e] = sum_d X[t][d] * Wg[d][e], bf16 inputs.
 * Each bf16 product is exact in double; the sum is accumulated in double.
 * ([p2] 1.2 names the gate/router network; the X*Wg form is the workload's.)
 */
void oracle_gate_logits(const uint16_t *X, const uint16_t *Wg, long long T,
                        long long d, long long E, double *logits)
{
    for (long long t = 0; t < T; ++t)
        for (long long e = 0; e < E; ++e) {
            double acc = 0.0;
            for (long long i = 0; i < d; ++i)
                acc += bf16_to_double(X[t * d + i]) * bf16_to_double(Wg[i * E + e]);
            logits[t * E + e] = acc;
        }
}

/*
 * Backward of the gate GEMM logits = X.Wg (bf16 inputs, see above):
 *   dX[t][i]  = sum_e dlogits[t][e] * Wg[i][e]      (dX  = dlogits . Wg^T)
 *   dWg[i][e] = sum_t X[t][i] * dlogits[t][e]       (dWg = X^T . dlogits)
 * in double; either output may be NULL.
 */
void oracle_gate_backward(const uint16_t *X, const uint16_t *Wg, const double *dlogits,
                          long long T, long long d, long long E, double *dX, double *dWg)
{
    if (dX)
        for (long long t = 0; t < T; ++t)
            for (long long i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long long e = 0; e < E; ++e)
                    acc += dlogits[t * E + e] * bf16_to_double(Wg[i * E + e]);
                dX[t * d + i] = acc;
            }
    if (dWg)
        for (long long i = 0; i < d; ++i)
            for (long long e = 0; e < E; ++e) {
                double acc = 0.0;
                for (long long t = 0; t < T; ++t)
                    acc += bf16_to_double(X[t * d + i]) * dlogits[t * E + e];
                dWg[i * E + e] = acc;
            }
}

/* Row softmax statistics: m = max_e l, s = sum_e exp(l - m). */
static void softmax_stats(const double *row, long long E, double *m_out, double *s_out)
{
    double m = row[0];
    for (long long e = 1; e < E; ++e)
        if (row[e] > m)
            m = row[e];
    double s = 0.0;
    for (long long e = 0; e < E; ++e)
        s += exp(row[e] - m);
    *m_out = m;
    *s_out = s;
}

/*
 * Top-k selection for one row: the first k experts in the order
 * (selection value descending, expert index ascending), where the selection
 * value is the logit itself or, with a selection bias, the biased logit.
 * Comparison is numeric, so -0.0 and +0.0 are equal and the lower index
 * wins.  Written as k passes of "take the best expert not taken yet"; a
 * strict '>' keeps the lowest index among equal values.
 */
static void topk_row(const double *row, long long E, long long k, int32_t *idx, char *taken)
{
    memset(taken, 0, (size_t)E);
    for (long long j = 0; j < k; ++j) {
        long long best = -1;
        for (long long e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || row[e] > row[best])
                best = e;
        }
        taken[best] = 1;
        idx[j] = (int32_t)best;
    }
}

/*
 * Forward routing of T tokens split into n_micro equal microbatches of
 * Tm = T / n_micro tokens; every microbatch is routed on its own.
 *
 * select_bias [E] (may be NULL): [p1] 4.3 adds a per-expert scalar b_i to
 * the router logits to steer the choice.  Reading: the bias enters the
 * selection only -- the gate weights, the probabilities behind P_i and the
 * aux loss keep the unbiased softmax -- and the biased value is the fp32 sum
 * l + b_i (the precision the logits and the bias are given in).
 *
 * p_masked: P_i from the picked positions only, as [p1] 4.4 codes it: the
 * softmax is zeroed outside each token's k picks and the sum is divided by
 * the number of assignments Tm*k (for k = 1 this is [p2] 3.1's masked mean
 * over tokens).  Otherwise P_i is the mean softmax over all tokens ([p1]
 * 4.2).  The picks are the pre-capacity top-k.
 *
 * Outputs (all caller-allocated; pointers marked "may be NULL" are skipped):
 *   topk_idx [T*k], topk_w [T*k]          selection and gate weights
 *   row_max, row_sum [T]      (may be NULL) softmax statistics
 *   counts   [m*E]             assignments per expert, before capacity
 *   offsets  [m*(E+1)]         exclusive scan of counts, local to the
 *                              microbatch's segment of perm
 *   perm     [T*k]             perm[m*Tm*k + pos] = flat index t*k+j
 *   inv_perm [T*k]  (may be NULL) inv_perm[t*k+j] = m*Tm*k + pos
 *   dropped  [T*k]             1 if the assignment is past capacity
 *   f, P     [m*E]             dispatch fraction and mean router probability
 *   aux, cv, max_over_mean [m]
 *   extra    [m*8]            min/mean, balance degree, entropy of f,
 *                              kept, dropped, capacity, max f, min f
 * Returns 0 on success, -1 on bad arguments.
 */
int oracle_route(const double *logits, long long T, long long E, long long k,
                 long long n_micro, long long capacity, double alpha, int renorm,
                 const float *select_bias, int p_masked, int32_t *topk_idx, double *topk_w, double *row_max, double *row_sum,
                 int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                 uint8_t *dropped, double *f, double *P, double *aux, double *cv,
                 double *max_over_mean, double *extra)
{
    if (T < 1 || E < 1 || k < 1 || k > E || n_micro < 1 || T % n_micro != 0)
        return -1;
    const long long Tm = T / n_micro;
    char *taken = (char *)malloc((size_t)E);
    double *psum = (double *)malloc(sizeof(double) * (size_t)E);
    long long *cursor = (long long *)malloc(sizeof(long long) * (size_t)E);
    double *selrow = (double *)malloc(sizeof(double) * (size_t)E);
    if (!taken || !psum || !cursor || !selrow) {
        free(taken); free(psum); free(cursor); free(selrow);
        return -1;
    }

    for (long long mb = 0; mb < n_micro; ++mb) {
        const long long t0 = mb * Tm;
        int32_t *cnt = counts + mb * E;
        int32_t *off = offsets + mb * (E + 1);
        for (long long e = 0; e < E; ++e) {
            cnt[e] = 0;
            psum[e] = 0.0;
        }

        /* Softmax, selection, gate weights; histogram and probability sums.
         * [p1] 4.2: p = softmax(router(x)); f counts the argmax/top-k picks,
         * P averages the softmax over all tokens of the batch.
         * [p1] 4.4 / [p2] 3.1: the histogram keeps zero-count experts. */
        for (long long t = t0; t < t0 + Tm; ++t) {
            const double *row = logits + t * E;
            double m, s;
            softmax_stats(row, E, &m, &s);
            if (row_max) row_max[t] = m;
            if (row_sum) row_sum[t] = s;
            if (!p_masked)
                for (long long e = 0; e < E; ++e)
                    psum[e] += exp(row[e] - m) / s;

            int32_t *idx = topk_idx + t * k;
            if (select_bias) {
                for (long long e = 0; e < E; ++e) {
                    float biased = (float)row[e] + select_bias[e];
                    selrow[e] = (double)biased;
                }
                topk_row(selrow, E, k, idx, taken);
            } else {
                topk_row(row, E, k, idx, taken);
            }
            double picked = 0.0;
            for (long long j = 0; j < k; ++j)
                picked += exp(row[idx[j]] - m) / s;
            for (long long j = 0; j < k; ++j) {
                double p = exp(row[idx[j]] - m) / s;
                /* Reading: with renorm the k picked probabilities are
                 * rescaled to sum to one; without it the gate is p itself. */
                topk_w[t * k + j] = renorm ? p / picked : p;
                cnt[idx[j]] += 1;
                if (p_masked)
                    psum[idx[j]] += p;
            }
        }

        /* Expert offsets: exclusive prefix sum of the counts. */
        off[0] = 0;
        for (long long e = 0; e < E; ++e)
            off[e + 1] = off[e] + cnt[e];

        /* Stable expert-sorted permutation with capacity drop.
         * Assignments are visited in (token, slot) order; the r-th one that
         * goes to expert e lands at off[e] + r and is dropped when r >= C.
         * ([p1] 4.5: tokens past an expert's capacity are dropped.) */
        for (long long e = 0; e < E; ++e)
            cursor[e] = 0;
        const long long seg = mb * Tm * k;
        for (long long t = t0; t < t0 + Tm; ++t)
            for (long long j = 0; j < k; ++j) {
                long long a = t * k + j;
                long long e = topk_idx[a];
                long long r = cursor[e]++;
                long long pos = off[e] + r;
                perm[seg + pos] = (int32_t)a;
                if (inv_perm) inv_perm[a] = (int32_t)(seg + pos);
                dropped[a] = (uint8_t)(capacity >= 0 && r >= capacity);
            }

        /* Statistics.  [p1] 4.2/4.4: f_i = count_i / (Tm*k),
         * P_i = mean softmax probability; aux = alpha * N * sum f_i * P_i.
         * [p3] 3.1/5.1: CV = std/mean over expert loads (population std),
         * load-balance degree = 1 - (max - mean)/mean.  [p1] 5.4: max/mean.
         * [p2] 4.2: max and min distribution ratio; entropy of the load. */
        const double total = (double)(Tm * k);
        const double mean = total / (double)E;
        double dot = 0.0, var = 0.0, ent = 0.0;
        double cmax = cnt[0], cmin = cnt[0];
        long long kept = 0;
        for (long long e = 0; e < E; ++e) {
            double fe = (double)cnt[e] / total;
            double pe = psum[e] / (p_masked ? total : (double)Tm);
            f[mb * E + e] = fe;
            P[mb * E + e] = pe;
            dot += fe * pe;
            var += ((double)cnt[e] - mean) * ((double)cnt[e] - mean);
            if (fe > 0.0)
                ent -= fe * log(fe);
            if (cnt[e] > cmax) cmax = cnt[e];
            if (cnt[e] < cmin) cmin = cnt[e];
            kept += (capacity >= 0 && cnt[e] > capacity) ? capacity : cnt[e];
        }
        var /= (double)E;
        aux[mb] = alpha * (double)E * dot;
        cv[mb] = sqrt(var) / mean;
        max_over_mean[mb] = cmax / mean;
        double *x = extra + mb * 8;
        x[0] = cmin / mean;
        x[1] = 1.0 - (cmax - mean) / mean;
        x[2] = ent;
        x[3] = (double)kept;
        x[4] = total - (double)kept;
        x[5] = (double)capacity;
        x[6] = cmax / total;
        x[7] = cmin / total;
    }
    free(taken);
    free(psum);
    free(cursor);
    free(selrow);
    return 0;
}

/*
 * Update of the selection bias after a forward pass.  [p1] 4.3: an
 * overloaded expert's b_i is pushed down, an idle one's up, and no loss term
 * is involved.  The page gives no step form; reading: a fixed step gamma
 * against the sign of the expert's load error, in fp32,
 *   load_e = sum over microbatches of counts[mb][e]  (pre-capacity),
 *   b_e <- b_e - gamma  if load_e > T*k/E,
 *   b_e <- b_e + gamma  if load_e < T*k/E,  unchanged if equal.
 * The comparison is done exactly in integers (load_e * E against T * k).
 */
void oracle_bias_update(const int32_t *counts, long long n_micro, long long E,
                        long long T, long long k, float gamma, float *bias)
{
    for (long long e = 0; e < E; ++e) {
        long long load = 0;
        for (long long mb = 0; mb < n_micro; ++mb)
            load += counts[mb * E + e];
        long long lhs = load * E, rhs = T * k;
        if (lhs > rhs)
            bias[e] = bias[e] - gamma;
        else if (lhs < rhs)
            bias[e] = bias[e] + gamma;
    }
}

/*
 * Gradient with respect to the logits of
 *   L = sum_mb g_mb * aux_mb + sum_{t,j} dW[t][j] * w[t][j]
 * with the selection (topk_idx) and the counts f held fixed ([p1] 4.2 and
 * [p2] 2.2: the routing choice and f_i are hard observations; the gradient
 * reaches the router through the probabilities only).
 *   aux_mb = alpha * E * sum_i f_i * P_i, P_i = (1/Tm) sum_t p[t][i], or with
 *   p_masked (([p1] 4.4) P_i = (1/(Tm*k)) sum_t m[t][i] p[t][i], m[t][i] = 1
 *   when i is one of t's picks;
 *   w[t][j] = p[t][idx_j], or p[t][idx_j] / sum_j' p[t][idx_j'] with renorm.
 * Written as the chain rule through the probabilities: for each token the
 * vector G_i = dL/dp[t][i] is formed from the two terms, then the softmax
 * Jacobian dp_i/dl_j = p_i (delta_ij - p_j) gives
 *   dL/dl[t][j] = p_j (G_j - sum_i G_i p_i).
 * g_mb is d_aux[mb] (1 if NULL); d_topk_w [T*k] may be NULL (no weight term).
 */
void oracle_backward(const double *logits, long long T, long long E, long long k,
                     long long n_micro, double alpha, const int32_t *counts,
                     const double *d_aux, int p_masked, const int32_t *topk_idx,
                     int renorm, const double *d_topk_w, double *dlogits)
{
    const long long Tm = T / n_micro;
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    double *G = (double *)malloc(sizeof(double) * (size_t)E);
    if (!p || !G) {
        free(p); free(G);
        return;
    }
    for (long long mb = 0; mb < n_micro; ++mb) {
        const double g = d_aux ? d_aux[mb] : 1.0;
        const int32_t *cnt = counts + mb * E;
        const double total = (double)(Tm * k);
        for (long long t = mb * Tm; t < (mb + 1) * Tm; ++t) {
            const double *row = logits + t * E;
            double m, s;
            softmax_stats(row, E, &m, &s);
            for (long long i = 0; i < E; ++i)
                p[i] = exp(row[i] - m) / s;
            /* aux term: dP_i/dp[t][i] = 1/Tm, or m[t][i]/(Tm*k) when masked */
            for (long long i = 0; i < E; ++i)
                G[i] = p_masked ? 0.0 : g * alpha * (double)E * ((double)cnt[i] / total) / (double)Tm;
            if (p_masked)
                for (long long j = 0; j < k; ++j) {
                    long long i = topk_idx[t * k + j];
                    G[i] += g * alpha * (double)E * ((double)cnt[i] / total) / total;
                }
            /* weight term */
            if (d_topk_w) {
                double z = 0.0;
                for (long long j = 0; j < k; ++j)
                    z += p[topk_idx[t * k + j]];
                for (long long j = 0; j < k; ++j) {
                    long long i = topk_idx[t * k + j];
                    if (!renorm) {
                        G[i] += d_topk_w[t * k + j]; /* w_j = p_i */
                    } else {
                        /* w_j = p_i / z: dw_j/dp_i = 1/z - p_i/z^2 and
                           dw_j'/dp_i = -p_idx_j'/z^2 for the other picks */
                        G[i] += d_topk_w[t * k + j] / z;
                        for (long long j2 = 0; j2 < k; ++j2)
                            G[i] -= d_topk_w[t * k + j2] * p[topk_idx[t * k + j2]] / (z * z);
                    }
                }
            }
            double gp = 0.0;
            for (long long i = 0; i < E; ++i)
                gp += G[i] * p[i];
            for (long long j = 0; j < E; ++j)
                dlogits[t * E + j] = p[j] * (G[j] - gp);
        }
    }
    free(p);
    free(G);
}

/*
 * EPLB placement ([p3] 4.1.2), global strategy: replicate, then pack.
 *
 * replicate_experts: every logical expert starts with one replica; while
 * the physical count is below num_phys, the expert with the largest load
 * per replica weight[e] / logcnt[e] gets one more.  Physical expert i < E
 * is logical i; replica E + r is the r-th copy made.  phy_rank[i] = the
 * replica's number within its expert (0 for the original).
 * balanced_packing: the physical replicas, weighted weight / logcnt of
 * their expert (final counts), are sorted by weight descending and placed
 * one by one into the lightest pack that holds fewer than
 * num_phys / num_packs items; slot = its position in the pack.
 * Readings: per-replica loads are compared exactly (cross-multiplied
 * integers); ties in the replication and in the sort go to the lower index,
 * ties between packs to the lower pack; pack loads are double sums
 * accumulated in placement order.  Returns 0, or -1 on bad arguments.
 */
struct eplb_item { long long num, den; long long idx; };

static int eplb_cmp_desc(const void *pa, const void *pb)
{
    const struct eplb_item *a = (const struct eplb_item *)pa;
    const struct eplb_item *b = (const struct eplb_item *)pb;
    long long l = a->num * b->den, r = b->num * a->den; /* a/b vs b's value */
    if (l != r) return l > r ? -1 : 1;
    return a->idx < b->idx ? -1 : (a->idx > b->idx ? 1 : 0);
}

int oracle_eplb(const int32_t *weight, long long E, long long num_phys, long long num_packs,
                int32_t *phy2log, int32_t *phy_rank, int32_t *logcnt, int32_t *pack,
                int32_t *slot, double *pack_load)
{
    if (E < 1 || num_phys < E || num_packs < 1 || num_phys % num_packs != 0)
        return -1;
    for (long long e = 0; e < E; ++e) {
        if (weight[e] < 0) return -1;
        phy2log[e] = (int32_t)e;
        phy_rank[e] = 0;
        logcnt[e] = 1;
    }
    for (long long i = E; i < num_phys; ++i) {
        long long best = 0;
        for (long long e = 1; e < E; ++e)
            if ((long long)weight[e] * logcnt[best] > (long long)weight[best] * logcnt[e])
                best = e;
        phy2log[i] = (int32_t)best;
        phy_rank[i] = logcnt[best];
        logcnt[best] += 1;
    }
    struct eplb_item *it = (struct eplb_item *)malloc(sizeof(struct eplb_item) * (size_t)num_phys);
    long long *cnt = (long long *)malloc(sizeof(long long) * (size_t)num_packs);
    if (!it || !cnt) {
        free(it); free(cnt);
        return -1;
    }
    for (long long i = 0; i < num_phys; ++i) {
        it[i].num = weight[phy2log[i]];
        it[i].den = logcnt[phy2log[i]];
        it[i].idx = i;
    }
    qsort(it, (size_t)num_phys, sizeof(struct eplb_item), eplb_cmp_desc);
    const long long cap = num_phys / num_packs;
    for (long long b = 0; b < num_packs; ++b) {
        cnt[b] = 0;
        pack_load[b] = 0.0;
    }
    for (long long n = 0; n < num_phys; ++n) {
        long long best = -1;
        for (long long b = 0; b < num_packs; ++b)
            if (cnt[b] < cap && (best < 0 || pack_load[b] < pack_load[best]))
                best = b;
        const long long i = it[n].idx;
        pack[i] = (int32_t)best;
        slot[i] = (int32_t)cnt[best];
        cnt[best] += 1;
        pack_load[best] += (double)it[n].num / (double)it[n].den;
    }
    free(it);
    free(cnt);
    return 0;
}

/*
 * Sinkhorn-Knopp flow plan ([p4] section 2, Phase 1).  supply a [R],
 * demand b [R] (a and b should carry the same total), cost C [R*R]
 * row-major, regularisation eps > 0.  Gibbs kernel K = exp(-C / eps);
 * starting from u = v = 1, each of the iters rounds sets
 *   u_i = a_i / max(sum_j K_ij v_j, tiny),  then
 *   v_j = b_j / max(sum_i K_ij u_i, tiny),
 * sums taken in index order, tiny = 1e-300 (the page's clamp; reading).
 * Outputs u [R], v [R] and the plan T [R*R], T_ij = u_i K_ij v_j.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_sinkhorn(const double *a, const double *b, const double *C, long long R, double eps,
                    long long iters, double *u, double *v, double *T)
{
    if (R < 1 || !(eps > 0.0) || iters < 0)
        return -1;
    double *K = (double *)malloc(sizeof(double) * (size_t)(R * R));
    if (!K)
        return -1;
    for (long long i = 0; i < R * R; ++i)
        K[i] = exp(-C[i] / eps);
    for (long long i = 0; i < R; ++i) {
        u[i] = 1.0;
        v[i] = 1.0;
    }
    const double tiny = 1e-300;
    for (long long it = 0; it < iters; ++it) {
        for (long long i = 0; i < R; ++i) {
            double s = 0.0;
            for (long long j = 0; j < R; ++j)
                s += K[i * R + j] * v[j];
            u[i] = a[i] / (s > tiny ? s : tiny);
        }
        for (long long j = 0; j < R; ++j) {
            double s = 0.0;
            for (long long i = 0; i < R; ++i)
                s += K[i * R + j] * u[i];
            v[j] = b[j] / (s > tiny ? s : tiny);
        }
    }
    for (long long i = 0; i < R; ++i)
        for (long long j = 0; j < R; ++j)
            T[i * R + j] = u[i] * K[i * R + j] * v[j];
    free(K);
    return 0;
}
