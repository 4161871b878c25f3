/*
 * moe_oracle.c -- CPU oracle for the MoE expert path (router -> dispatch ->
 * grouped GEMM1 -> SwiGLU -> grouped GEMM2 -> weighted combine, and the
 * backward of all of it).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it follows (page "MegaMoE", Primus technical guide):
 *   - intro: fused router = score function + group-limited top-k + aux score;
 *     expert path = dispatch -> GEMM1 -> SwiGLU -> GEMM2 -> combine with a
 *     weighted reduce; the load-balancing aux loss is returned.
 *   - "Design: two stages + weight modules": w1 is [g, 2I, H] holding gate
 *     rows then up rows, w2 is [g, H, I]; backward yields dW2, then dW1.
 *   - "Required" settings: gated SwiGLU with SiLU, no bias in the linears.
 *   - "Router force load balancing": the `even` routing formula (a test pin).
 * SwiGLU itself is silu(x_glu) * x_linear (page "GDN <-> FLA Parity in
 * Primus", "What changed and why", table B, the fused-SwiGLU patch row), with
 * x_glu the gate half.
 *
 * Precision: every value on the expert path is computed in double from the
 * exact (bf16 / fp32) inputs; nothing is rounded to bf16 in between.  The one
 * place floating point decides an integer -- the top-k -- takes its decision
 * on an fp32 score tensor, as the GPU path does.  Readings where the pages are
 * silent (tie rules, group score, aux formula, sigmoid weight scaling, bias
 * use) are stated at each function.
 *
 * Everything is written as the plain definition: per-token loops over the
 * selected experts, no blocking, no fusion.  OpenMP splits only independent
 * outer iterations (tokens, or experts for the weight gradients).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_SOFTMAX 0
#define OR_SIGMOID 1

/* bf16 bit pattern -> exact double (bf16 is the top half of an fp32). */
static double bf(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double z) { return z * sigmoid(z); }

/* ------------------------------------------------------------------------ */
/* Router projection: l[t,e] = sum_h x[t,h] * Wr[e,h]  (Wr is [E,H], fp32).   */
/* Output in double; callers round to fp32 when they need the fp32 logits.   */
/* ------------------------------------------------------------------------ */
void oracle_logits(int64_t T, int32_t H, int32_t E, const uint16_t *x,
                   const float *Wr, double *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h)
                acc += bf(x[t * H + h]) * (double)Wr[(int64_t)e * H + h];
            logits[t * E + e] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Selection scores S (fp32), the tensor the top-k decides on.               */
/*   softmax router: S = l  (softmax is strictly increasing, so the top-k of  */
/*                   the probabilities is the top-k of the logits; deciding  */
/*                   on l avoids ties created by rounding exp).               */
/*   sigmoid router: S = fp32(sigmoid(l)) + b, an fp32 add; b (nullable) is  */
/*                   a per-expert bias that takes part in selection only.    */
/* logits are the fp32 logits.                                               */
/* ------------------------------------------------------------------------ */
void oracle_selection_scores(int64_t T, int32_t E, int32_t score,
                             const float *logits, const float *bias, float *S)
{
    for (int64_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) {
            float l = logits[t * E + e];
            if (score == OR_SOFTMAX) {
                S[t * E + e] = l;
            } else {
                float s = (float)sigmoid((double)l);
                float b = bias ? bias[e] : 0.0f;
                S[t * E + e] = s + b;
            }
        }
}

/* The ranking key of a selection score: the score itself, with NaN taken as
   -inf (reading: the pages rank scores only; a NaN score ranks below every
   number, ties by lower index as for any equal scores). */
static float sel_key(float v) { return isnan(v) ? -INFINITY : v; }

/* a ranks before b: larger key first, equal keys -> lower index first. */
static int ranks_before(float va, int32_t ia, float vb, int32_t ib)
{
    va = sel_key(va);
    vb = sel_key(vb);
    return va > vb || (va == vb && ia < ib);
}

/* ------------------------------------------------------------------------ */
/* Group-limited top-k on fp32 scores S [T,E] -> idx [T,k].                   */
/*   G groups of E/G contiguous experts (reading: contiguous blocks).        */
/*   If G > 1: group score = sum (fp32 add) of the two largest S in the      */
/*   group (just the largest when a group has one expert); the kg best       */
/*   groups are kept (ties -> lower group index); only their experts are     */
/*   eligible.  Then the k best eligible experts, best first (ties -> lower  */
/*   expert index).  Selection is by repeated arg-max.                       */
/* ------------------------------------------------------------------------ */
void oracle_topk(int64_t T, int32_t E, int32_t k, int32_t G, int32_t kg,
                 const float *S, int32_t *idx)
{
#pragma omp parallel
    {
        unsigned char *eligible = (unsigned char *)malloc((size_t)E);
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
        float *gs = (float *)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
        unsigned char *gtaken = (unsigned char *)malloc((size_t)(G > 0 ? G : 1));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float *s = S + t * E;
            if (G > 1) {
                int32_t gsz = E / G;
                for (int32_t g = 0; g < G; ++g) {
                    int32_t best = -1, second = -1;
                    for (int32_t e = g * gsz; e < (g + 1) * gsz; ++e)
                        if (best < 0 || ranks_before(s[e], e, s[best], best))
                            best = e;
                    for (int32_t e = g * gsz; e < (g + 1) * gsz; ++e)
                        if (e != best &&
                            (second < 0 || ranks_before(s[e], e, s[second], second)))
                            second = e;
                    gs[g] = sel_key((second >= 0) ? sel_key(s[best]) + sel_key(s[second])
                                                  : sel_key(s[best]));
                    gtaken[g] = 0;
                }
                for (int32_t e = 0; e < E; ++e) eligible[e] = 0;
                for (int32_t r = 0; r < kg; ++r) {
                    int32_t bg = -1;
                    for (int32_t g = 0; g < G; ++g)
                        if (!gtaken[g] && (bg < 0 || ranks_before(gs[g], g, gs[bg], bg)))
                            bg = g;
                    gtaken[bg] = 1;
                    for (int32_t e = bg * gsz; e < (bg + 1) * gsz; ++e) eligible[e] = 1;
                }
            } else {
                for (int32_t e = 0; e < E; ++e) eligible[e] = 1;
            }
            for (int32_t e = 0; e < E; ++e) taken[e] = 0;
            for (int32_t j = 0; j < k; ++j) {
                int32_t be = -1;
                for (int32_t e = 0; e < E; ++e)
                    if (eligible[e] && !taken[e] &&
                        (be < 0 || ranks_before(s[e], e, s[be], be)))
                        be = e;
                taken[be] = 1;
                idx[t * k + j] = be;
            }
        }
        free(eligible);
        free(taken);
        free(gs);
        free(gtaken);
    }
}

/* ------------------------------------------------------------------------ */
/* `even` forced routing (MegaMoE page, "Router force load balancing",      */
/* table row `even`): the router's choice is discarded and slot j of token  */
/* t goes to expert (t * k + j) mod E, so every expert gets the same number */
/* of slots (to within one).  Weights, counts and aux then follow from      */
/* these indices exactly as for a learned choice.                           */
/* ------------------------------------------------------------------------ */
void oracle_even_topk(int64_t T, int32_t E, int32_t k, int32_t *idx)
{
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) idx[t * k + j] = (int32_t)((t * k + j) % E);
}

/* Router probabilities of one token over all E experts (double):            */
/*   softmax router: p = softmax(l);  sigmoid router: s = sigmoid(l).        */
static void token_scores(int32_t E, int32_t score, const double *l, double *out)
{
    if (score == OR_SOFTMAX) {
        double m = l[0];
        for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
        double z = 0.0;
        for (int32_t e = 0; e < E; ++e) { out[e] = exp(l[e] - m); z += out[e]; }
        for (int32_t e = 0; e < E; ++e) out[e] /= z;
    } else {
        for (int32_t e = 0; e < E; ++e) out[e] = sigmoid(l[e]);
    }
}

/* ------------------------------------------------------------------------ */
/* Routing weights w [T,k] (double) for given indices.                       */
/*   softmax: w_j = p[idx_j], divided by sum_j p[idx_j] when renorm != 0.    */
/*   sigmoid: w_j = scale * s[idx_j] / sum_j s[idx_j]  (normalised, then     */
/*            scaled); the selection bias never enters the weights.          */
/* ------------------------------------------------------------------------ */
void oracle_weights(int64_t T, int32_t E, int32_t k, int32_t score,
                    int32_t renorm, double scale, const double *logits,
                    const int32_t *idx, double *w)
{
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            token_scores(E, score, logits + t * E, p);
            double z = 0.0;
            for (int32_t j = 0; j < k; ++j) z += p[idx[t * k + j]];
            for (int32_t j = 0; j < k; ++j) {
                double v = p[idx[t * k + j]];
                if (score == OR_SOFTMAX)
                    w[t * k + j] = renorm ? v / z : v;
                else
                    w[t * k + j] = scale * v / z;
            }
        }
        free(p);
    }
}

/* ------------------------------------------------------------------------ */
/* Dispatch bookkeeping.  Flat slot f = t*k + j.                             */
/*   counts[e]  = number of slots routed to e                                */
/*   offsets    = exclusive prefix sum of counts, offsets[E] = T*k           */
/*   row_map[r] = the flat slot placed at sorted row r: experts in ascending */
/*                order, and inside one expert ascending flat slot (stable)  */
/*   pos[f]     = the sorted row of flat slot f (inverse of row_map)         */
/* ------------------------------------------------------------------------ */
void oracle_permute(int64_t T, int32_t k, int32_t E, const int32_t *idx,
                    int32_t *counts, int32_t *offsets, int32_t *row_map,
                    int32_t *pos)
{
    int64_t M = T * k;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t f = 0; f < M; ++f) counts[idx[f]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t r = 0;
    for (int32_t e = 0; e < E; ++e)
        for (int64_t f = 0; f < M; ++f)
            if (idx[f] == e) {
                row_map[r] = (int32_t)f;
                pos[f] = (int32_t)r;
                ++r;
            }
}

/* ------------------------------------------------------------------------ */
/* Load-balancing aux loss (reading; the pages give no formula):             */
/*   aux = coeff * E / (k * T^2) * sum_e counts[e] * sum_t p[t,e]            */
/* = coeff * E * sum_e f_e * P_e with f_e = counts[e]/(k T), P_e = mean_t p. */
/* p = softmax(l) for the softmax router, s / sum_e s for the sigmoid one.  */
/* ------------------------------------------------------------------------ */
double oracle_aux(int64_t T, int32_t E, int32_t k, int32_t score, double coeff,
                  const double *logits, const int32_t *counts)
{
    if (T == 0) return 0.0;
    double *P = (double *)calloc((size_t)E, sizeof(double));
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        token_scores(E, score, logits + t * E, p);
        if (score == OR_SIGMOID) {
            double z = 0.0;
            for (int32_t e = 0; e < E; ++e) z += p[e];
            for (int32_t e = 0; e < E; ++e) p[e] /= z;
        }
        for (int32_t e = 0; e < E; ++e) P[e] += p[e];
    }
    double acc = 0.0;
    for (int32_t e = 0; e < E; ++e) acc += (double)counts[e] * P[e];
    free(P);
    free(p);
    return coeff * (double)E / ((double)k * (double)T * (double)T) * acc;
}

/* One (token, expert) pair of the expert MLP, forward:                     */
/*   g[i] = sum_h x[h] w1[e,i,h],  u[i] = sum_h x[h] w1[e,I+i,h]             */
/*   a[i] = silu(g[i]) * u[i],     o[h] = sum_i w2[e,h,i] a[i]               */
static void expert_mlp(int32_t H, int32_t I, const uint16_t *xt,
                       const uint16_t *w1e, const uint16_t *w2e, double *g,
                       double *u, double *a, double *o)
{
    for (int32_t i = 0; i < I; ++i) {
        double sg = 0.0, su = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            double xv = bf(xt[h]);
            sg += xv * bf(w1e[(int64_t)i * H + h]);
            su += xv * bf(w1e[(int64_t)(I + i) * H + h]);
        }
        g[i] = sg;
        u[i] = su;
        a[i] = silu(sg) * su;
    }
    if (o)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t i = 0; i < I; ++i) acc += bf(w2e[(int64_t)h * I + i]) * a[i];
            o[h] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Expert forward for a list of tokens (toks == NULL: tokens 0..ntok-1).     */
/*   y[t] = sum_{j=0..k-1} w[t,j] * o(t, idx[t,j])   (j ascending)           */
/* x [T,H] bf16, w1 [E,2I,H] bf16, w2 [E,H,I] bf16, y [ntok,H] double.       */
/* ------------------------------------------------------------------------ */
void oracle_forward(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                    const uint16_t *x, const uint16_t *w1, const uint16_t *w2,
                    const int32_t *idx, const double *w, int64_t ntok,
                    const int64_t *toks, double *y)
{
    (void)T;
    (void)E;
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            int64_t t = toks ? toks[n] : n;
            double *yt = y + n * H;
            for (int32_t h = 0; h < H; ++h) yt[h] = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = idx[t * k + j];
                expert_mlp(H, I, x + t * H, w1 + (int64_t)e * 2 * I * H,
                           w2 + (int64_t)e * H * I, g, u, a, o);
                for (int32_t h = 0; h < H; ++h) yt[h] += w[t * k + j] * o[h];
            }
        }
        free(g);
        free(u);
        free(a);
        free(o);
    }
}

/* Router part of the backward for one token, given the gradient dw[j] of  */
/* the loss w.r.t. each routing weight (the expert path's row-dots):        */
/*   softmax: dp at selected e_j = renorm ? (dw_j - sum dw w)/sum p_sel      */
/*                                        : dw_j                             */
/*            plus aux: d_aux*coeff*E/(k T^2)*counts[e] at every e;         */
/*            dl = p * (dp - <dp, p>)                                        */
/*   sigmoid: ds at selected e_j = scale/sum s_sel * (dw_j - sum dw w/scale) */
/*            plus aux through p = s/sum s: (a_e - sum a p)/sum s;           */
/*            dl = ds * s * (1 - s)                                          */
/*   dxt += sum_e dl[e] Wr[e,:]   (when Wr != NULL)                          */
/* lt: the token's logits [E]; it: its experts [k]; wt: scratch [k];        */
/* p, dp: scratch [E].                                                       */
static void router_token_backward(int64_t T, int32_t H, int32_t E, int32_t k, int32_t score,
                                  int32_t renorm, double scale, double coeff, double d_aux,
                                  const float *Wr, const double *lt, const int32_t *it,
                                  const int32_t *counts, const double *dw, double *wt,
                                  double *p, double *dp, double *dl, double *dxt)
{
    token_scores(E, score, lt, p);
    double zsel = 0.0;
    for (int32_t j = 0; j < k; ++j) zsel += p[it[j]];
    for (int32_t j = 0; j < k; ++j) {
        double v = p[it[j]];
        if (score == OR_SOFTMAX) wt[j] = renorm ? v / zsel : v;
        else wt[j] = scale * v / zsel;
    }
    double sdw = 0.0;
    for (int32_t j = 0; j < k; ++j) sdw += dw[j] * wt[j];
    for (int32_t e = 0; e < E; ++e) dp[e] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
        int32_t e = it[j];
        if (score == OR_SOFTMAX)
            dp[e] += renorm ? (dw[j] - sdw) / zsel : dw[j];
        else
            dp[e] += scale / zsel * (dw[j] - sdw / scale);
    }
    double aux_scale = (T > 0) ? d_aux * coeff * (double)E /
                                     ((double)k * (double)T * (double)T)
                               : 0.0;
    if (score == OR_SOFTMAX) {
        for (int32_t e = 0; e < E; ++e) dp[e] += aux_scale * (double)counts[e];
        double dot = 0.0;
        for (int32_t e = 0; e < E; ++e) dot += dp[e] * p[e];
        for (int32_t e = 0; e < E; ++e) dl[e] = p[e] * (dp[e] - dot);
    } else {
        double q = 0.0;
        for (int32_t e = 0; e < E; ++e) q += p[e];
        double ap = 0.0;
        for (int32_t e = 0; e < E; ++e) ap += aux_scale * (double)counts[e] * (p[e] / q);
        for (int32_t e = 0; e < E; ++e)
            dp[e] += (aux_scale * (double)counts[e] - ap) / q;
        for (int32_t e = 0; e < E; ++e) dl[e] = dp[e] * p[e] * (1.0 - p[e]);
    }
    if (Wr)
        for (int32_t e = 0; e < E; ++e)
            for (int32_t h = 0; h < H; ++h)
                dxt[h] += dl[e] * (double)Wr[(int64_t)e * H + h];
}

/* ------------------------------------------------------------------------ */
/* Backward for a list of tokens: dx [ntok,H] and dlogits [ntok,E] (double). */
/* Loss = sum_t <dy[t], y[t]> + d_aux * aux.                                 */
/* Per slot (t,j), e = idx[t,j]:                                             */
/*   dw_j  = <dy_t, o>                                                       */
/*   dA_i  = w_j * sum_h w2[e,h,i] dy_t[h]                                   */
/*   dg_i  = dA_i * u_i * sig(g_i) * (1 + g_i (1 - sig(g_i)))                */
/*   du_i  = dA_i * silu(g_i)                                                */
/*   dx_t += sum_i (w1[e,i,:] dg_i + w1[e,I+i,:] du_i)                       */
/* Router (counts are constants, the selection carries no gradient):        */
/*   softmax: dp at selected e_j = renorm ? (dw_j - sum dw w)/sum p_sel      */
/*                                        : dw_j                             */
/*            plus aux: d_aux*coeff*E/(k T^2)*counts[e] at every e;         */
/*            dl = p * (dp - <dp, p>)                                        */
/*   sigmoid: ds at selected e_j = scale/sum s_sel * (dw_j - sum dw w/scale) */
/*            plus aux through p = s/sum s: (a_e - sum a p)/sum s;           */
/*            dl = ds * s * (1 - s)                                          */
/*   dx_t += sum_e dl[e] Wr[e,:]   (when Wr != NULL)                         */
/* logits are the router logits in double, counts the routed counts.        */
/* ------------------------------------------------------------------------ */
void oracle_backward_tokens(int64_t T, int32_t H, int32_t I, int32_t E,
                            int32_t k, int32_t score, int32_t renorm,
                            double scale, double coeff, double d_aux,
                            const uint16_t *x, const float *Wr,
                            const double *logits, const uint16_t *w1,
                            const uint16_t *w2, const int32_t *idx,
                            const int32_t *counts, const uint16_t *dy,
                            int64_t ntok, const int64_t *toks, double *dx,
                            double *dlogits)
{
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        double *dp = (double *)malloc(sizeof(double) * (size_t)E);
        double *wt = (double *)malloc(sizeof(double) * (size_t)k);
        double *dw = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            int64_t t = toks ? toks[n] : n;
            const uint16_t *xt = x + t * H;
            const uint16_t *dyt = dy + t * H;
            double *dxt = dx + n * H;
            for (int32_t h = 0; h < H; ++h) dxt[h] = 0.0;

            /* routing weights of this token */
            token_scores(E, score, logits + t * E, p);
            double zsel = 0.0;
            for (int32_t j = 0; j < k; ++j) zsel += p[idx[t * k + j]];
            for (int32_t j = 0; j < k; ++j) {
                double v = p[idx[t * k + j]];
                if (score == OR_SOFTMAX) wt[j] = renorm ? v / zsel : v;
                else wt[j] = scale * v / zsel;
            }

            for (int32_t j = 0; j < k; ++j) {
                int32_t e = idx[t * k + j];
                const uint16_t *w1e = w1 + (int64_t)e * 2 * I * H;
                const uint16_t *w2e = w2 + (int64_t)e * H * I;
                expert_mlp(H, I, xt, w1e, w2e, g, u, a, o);
                double acc = 0.0;
                for (int32_t h = 0; h < H; ++h) acc += bf(dyt[h]) * o[h];
                dw[j] = acc;
                for (int32_t i = 0; i < I; ++i) {
                    double dA = 0.0;
                    for (int32_t h = 0; h < H; ++h)
                        dA += bf(w2e[(int64_t)h * I + i]) * bf(dyt[h]);
                    dA *= wt[j];
                    double sg = sigmoid(g[i]);
                    double dg = dA * u[i] * sg * (1.0 + g[i] * (1.0 - sg));
                    double du = dA * silu(g[i]);
                    for (int32_t h = 0; h < H; ++h)
                        dxt[h] += bf(w1e[(int64_t)i * H + h]) * dg +
                                  bf(w1e[(int64_t)(I + i) * H + h]) * du;
                }
            }

            /* router */
            router_token_backward(T, H, E, k, score, renorm, scale, coeff, d_aux, Wr,
                                  logits + t * E, idx + t * k, counts, dw, wt, p, dp,
                                  dlogits + n * E, dxt);
        }
        free(g);
        free(u);
        free(a);
        free(o);
        free(p);
        free(dp);
        free(wt);
        free(dw);
    }
}

/* ------------------------------------------------------------------------ */
/* Expert weight gradients for a list of experts (experts == NULL: 0..ne-1), */
/* summed over the listed tokens (toks == NULL: all T tokens):               */
/*   dW2[e,h,i]   = sum_{(t,j): idx=e} w_tj dy_t[h] a_i                      */
/*   dW1[e,i,h]   = sum dg_i x_t[h],   dW1[e,I+i,h] = sum du_i x_t[h]        */
/* dW1 [ne,2I,H], dW2 [ne,H,I] in double, overwritten.  w [T,k] double.     */
/* ------------------------------------------------------------------------ */
void oracle_weight_grads(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                         const uint16_t *x, const uint16_t *w1,
                         const uint16_t *w2, const int32_t *idx,
                         const double *w, const uint16_t *dy, int32_t ne,
                         const int32_t *experts, int64_t ntok,
                         const int64_t *toks, double *dW1, double *dW2)
{
    (void)E;
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int32_t q = 0; q < ne; ++q) {
            int32_t e = experts ? experts[q] : q;
            const uint16_t *w1e = w1 + (int64_t)e * 2 * I * H;
            const uint16_t *w2e = w2 + (int64_t)e * H * I;
            double *d1 = dW1 + (int64_t)q * 2 * I * H;
            double *d2 = dW2 + (int64_t)q * H * I;
            memset(d1, 0, sizeof(double) * (size_t)2 * I * H);
            memset(d2, 0, sizeof(double) * (size_t)H * I);
            int64_t nt = toks ? ntok : T;
            for (int64_t n = 0; n < nt; ++n) {
                int64_t t = toks ? toks[n] : n;
                for (int32_t j = 0; j < k; ++j) {
                    if (idx[t * k + j] != e) continue;
                    const uint16_t *xt = x + t * H;
                    const uint16_t *dyt = dy + t * H;
                    double wj = w[t * k + j];
                    expert_mlp(H, I, xt, w1e, w2e, g, u, a, NULL);
                    for (int32_t h = 0; h < H; ++h) {
                        double c = wj * bf(dyt[h]);
                        for (int32_t i = 0; i < I; ++i) d2[(int64_t)h * I + i] += c * a[i];
                    }
                    for (int32_t i = 0; i < I; ++i) {
                        double dA = 0.0;
                        for (int32_t h = 0; h < H; ++h)
                            dA += bf(w2e[(int64_t)h * I + i]) * bf(dyt[h]);
                        dA *= wj;
                        double sg = sigmoid(g[i]);
                        double dg = dA * u[i] * sg * (1.0 + g[i] * (1.0 - sg));
                        double du = dA * silu(g[i]);
                        for (int32_t h = 0; h < H; ++h) {
                            double xv = bf(xt[h]);
                            d1[(int64_t)i * H + h] += dg * xv;
                            d1[(int64_t)(I + i) * H + h] += du * xv;
                        }
                    }
                }
            }
        }
        free(g);
        free(u);
        free(a);
    }
}

/* ------------------------------------------------------------------------ */
/* Single elements of dW1 / dW2 (for full-size shapes, where whole weight    */
/* gradients are out of reach on the CPU).  Element q is                     */
/*   which[q] == 1: dW1[ee[q], rr[q], cc[q]]   (row n < 2I, column h)        */
/*   which[q] == 2: dW2[ee[q], rr[q], cc[q]]   (row h, column i)             */
/* summed over all T tokens; same definitions as oracle_weight_grads.        */
/* ------------------------------------------------------------------------ */
void oracle_weight_grad_elements(int64_t T, int32_t H, int32_t I, int32_t k,
                                 const uint16_t *x, const uint16_t *w1,
                                 const uint16_t *w2, const int32_t *idx,
                                 const double *w, const uint16_t *dy,
                                 int64_t nel, const int32_t *which,
                                 const int32_t *ee, const int32_t *rr,
                                 const int32_t *cc, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nel; ++q) {
        int32_t e = ee[q];
        const uint16_t *w1e = w1 + (int64_t)e * 2 * I * H;
        const uint16_t *w2e = w2 + (int64_t)e * H * I;
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t)
            for (int32_t j = 0; j < k; ++j) {
                if (idx[t * k + j] != e) continue;
                const uint16_t *xt = x + t * H;
                const uint16_t *dyt = dy + t * H;
                double wj = w[t * k + j];
                int32_t i = (which[q] == 2) ? cc[q] : (rr[q] % I);
                double sg_, su_;
                {
                    double s1 = 0.0, s2 = 0.0;
                    for (int32_t h = 0; h < H; ++h) {
                        double xv = bf(xt[h]);
                        s1 += xv * bf(w1e[(int64_t)i * H + h]);
                        s2 += xv * bf(w1e[(int64_t)(I + i) * H + h]);
                    }
                    sg_ = s1;
                    su_ = s2;
                }
                if (which[q] == 2) {
                    double ai = silu(sg_) * su_;
                    acc += wj * bf(dyt[rr[q]]) * ai;
                } else {
                    double dA = 0.0;
                    for (int32_t h = 0; h < H; ++h)
                        dA += bf(w2e[(int64_t)h * I + i]) * bf(dyt[h]);
                    dA *= wj;
                    double sg = sigmoid(sg_);
                    double d = (rr[q] < I) ? dA * su_ * sg * (1.0 + sg_ * (1.0 - sg))
                                           : dA * silu(sg_);
                    acc += d * bf(xt[cc[q]]);
                }
            }
        out[q] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Whole lines of the expert weight gradients, each H long (for full-size    */
/* shapes: a few lines per expert reach every output tile of its gradient):  */
/*   which[q] == 1: out[q, h] = dW1[ee[q], rr[q], h]   (a row, n = rr[q])    */
/*   which[q] == 2: out[q, h] = dW2[ee[q], h, rr[q]]   (a column, i = rr[q]) */
/* summed over all T tokens; same definitions as oracle_weight_grads:       */
/*   dW1[e,i,h] = sum dg_i x_t[h], dW1[e,I+i,h] = sum du_i x_t[h],           */
/*   dW2[e,h,i] = sum w_tj dy_t[h] a_i, over the slots (t,j) with idx = e.   */
/* out [nl, H] double, overwritten.                                          */
/* ------------------------------------------------------------------------ */
void oracle_weight_grad_lines(int64_t T, int32_t H, int32_t I, int32_t k,
                              const uint16_t *x, const uint16_t *w1,
                              const uint16_t *w2, const int32_t *idx,
                              const double *w, const uint16_t *dy, int64_t nl,
                              const int32_t *which, const int32_t *ee,
                              const int32_t *rr, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nl; ++q) {
        const int32_t e = ee[q];
        const uint16_t *w1e = w1 + (int64_t)e * 2 * I * H;
        const uint16_t *w2e = w2 + (int64_t)e * H * I;
        const int32_t i = (which[q] == 2) ? rr[q] : (rr[q] % I);
        double *line = out + q * H;
        for (int32_t h = 0; h < H; ++h) line[h] = 0.0;
        for (int64_t t = 0; t < T; ++t)
            for (int32_t j = 0; j < k; ++j) {
                if (idx[t * k + j] != e) continue;
                const uint16_t *xt = x + t * H;
                const uint16_t *dyt = dy + t * H;
                const double wj = w[t * k + j];
                double g = 0.0, u = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    double xv = bf(xt[h]);
                    g += xv * bf(w1e[(int64_t)i * H + h]);
                    u += xv * bf(w1e[(int64_t)(I + i) * H + h]);
                }
                if (which[q] == 2) {
                    const double ai = silu(g) * u;
                    for (int32_t h = 0; h < H; ++h) line[h] += wj * bf(dyt[h]) * ai;
                } else {
                    double dA = 0.0;
                    for (int32_t h = 0; h < H; ++h)
                        dA += bf(w2e[(int64_t)h * I + i]) * bf(dyt[h]);
                    dA *= wj;
                    const double sg = sigmoid(g);
                    const double d = (rr[q] < I) ? dA * u * sg * (1.0 + g * (1.0 - sg))
                                                 : dA * silu(g);
                    for (int32_t h = 0; h < H; ++h) line[h] += d * bf(xt[h]);
                }
            }
    }
}

/* ------------------------------------------------------------------------ */
/* Router weight gradient: dWr[e,h] = sum_t dlogits[t,e] x[t,h]  (double).   */
/* ------------------------------------------------------------------------ */
void oracle_router_weight_grad(int64_t T, int32_t H, int32_t E,
                               const uint16_t *x, const double *dlogits,
                               double *dWr)
{
#pragma omp parallel for schedule(static)
    for (int32_t e = 0; e < E; ++e)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t) acc += dlogits[t * E + e] * bf(x[t * H + h]);
            dWr[(int64_t)e * H + h] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Per-slot intermediates of the expert MLP for listed flat slots f = t*k+j  */
/* (e = idx[f]): g [n,I], u [n,I], a [n,I], o [n,H] in double, where         */
/* g, u are the gate / up halves of x_t . w1[e]^T, a = silu(g) * u and       */
/* o = a . w2[e]^T (the expert output before the routing weight).           */
/* ------------------------------------------------------------------------ */
void oracle_expert_rows(int32_t H, int32_t I, int32_t k, const uint16_t *x,
                        const uint16_t *w1, const uint16_t *w2,
                        const int32_t *idx, int64_t n, const int64_t *slots,
                        double *g, double *u, double *a, double *o)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n; ++q) {
        int64_t f = slots[q];
        int64_t t = f / k;
        int32_t e = idx[f];
        expert_mlp(H, I, x + t * H, w1 + (int64_t)e * 2 * I * H,
                   w2 + (int64_t)e * H * I, g + q * I, u + q * I, a + q * I,
                   o + q * H);
    }
}

/* ======================================================================== */
/* MXFP8 expert precision (page "MegaMoE", "Expert precision": the two      */
/* expert stages run in MXFP8).  The pages name the format only; MXFP8 is    */
/* read as the OCP Microscaling (MX) v1.0 format:                           */
/*   - a block is 32 consecutive elements along the contraction dimension;   */
/*   - the block shares one E8M0 scale 2^X, X = floor(log2(amax)) - 8, where */
/*     8 is the exponent of E4M3's largest normal (448 = 1.75 * 2^8); X is   */
/*     clamped to E8M0's range [-127, 127]; an all-zero block takes X = -127;*/
/*   - each element is v / 2^X rounded to nearest-even E4M3, saturating to   */
/*     +-448 (E4M3 has no infinity; 0x7F / 0xFF are NaN and never produced). */
/* E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0   */
/* is subnormal, m * 2^-9.                                                   */
/* ======================================================================== */

double oracle_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Nearest-even E4M3 code of q (already divided by the block scale),         */
/* saturating.  The grid spacing around |q| is 2^(max(floor(log2|q|),-6)-3). */
static uint8_t e4m3_encode(double q)
{
    int neg = signbit(q) ? 1 : 0, ex, e, m;
    double a = fabs(q), step, r;
    if (a == 0.0) return (uint8_t)(neg << 7);
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
    e = ex - 1;
    if (e < -6) e = -6;
    step = ldexp(1.0, e - 3);
    r = nearbyint(a / step) * step; /* a / step is exact; ties to even */
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return (uint8_t)(neg << 7);
    if (r < ldexp(1.0, -6)) {
        m = (int)ldexp(r, 9); /* subnormal: r = m * 2^-9 */
        return (uint8_t)((neg << 7) | m);
    }
    frexp(r, &ex);
    e = ex - 1;
    m = (int)((ldexp(r, -e) - 1.0) * 8.0);
    return (uint8_t)((neg << 7) | ((e + 7) << 3) | m);
}

/* One block of n values (n = 32): scale code X + 127 and the element codes. */
static uint8_t mx_block(const double *v, int n, uint8_t *codes)
{
    double amax = 0.0;
    int X, ex, i;
    for (i = 0; i < n; ++i)
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) {
        X = -127;
    } else {
        frexp(amax, &ex);
        X = (ex - 1) - 8;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    for (i = 0; i < n; ++i) codes[i] = e4m3_encode(ldexp(v[i], -X));
    return (uint8_t)(X + 127);
}

static double mx_scale(uint8_t s) { return ldexp(1.0, (int)s - 127); }

/* Row-wise MXFP8 quantisation of a bf16 matrix src [rows, K] (K a multiple  */
/* of 32): codes [rows, K], scales [rows, K/32] (block b of row r covers     */
/* columns 32b .. 32b+31).                                                   */
void oracle_mx_quantize(int64_t rows, int64_t K, const uint16_t *src, uint8_t *codes,
                        uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[32];
        for (int64_t b = 0; b < K / 32; ++b) {
            for (int i = 0; i < 32; ++i) v[i] = bf(src[r * K + b * 32 + i]);
            scales[r * (K / 32) + b] = mx_block(v, 32, codes + r * K + b * 32);
        }
    }
}

/* The value an MX element stands for: E4M3 value times the block scale.    */
static double mx_value(const uint8_t *codes, const uint8_t *scales, int64_t K, int64_t r,
                       int64_t c)
{
    return oracle_e4m3_value(codes[r * K + c]) * mx_scale(scales[r * (K / 32) + c / 32]);
}

/* fp32 -> bf16, nearest-even (finite values). */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* One (token, expert) slot of the MXFP8 expert MLP.  Operands are MX        */
/* matrices quantised along their contraction dimension:                    */
/*   x  [T, H]      (blocks along H)     w1 [E*2I, H] (blocks along H)      */
/*   w2 [E*H, I]    (blocks along I)                                        */
/*   g, u = gate / up halves of X . W1[e]^T (double, from the MX values)     */
/*   a    = silu(g) * u, then rounded to fp32 and to bf16 (the precision in  */
/*          which the path holds its activations) and MX-quantised along I   */
/*          into aq [I], as_ [I/32]                                          */
/*   o    = A . W2[e]^T from the MX values of a                              */
static void mx_slot(int32_t H, int32_t I, int64_t t, int32_t e, const uint8_t *xq,
                    const uint8_t *xs, const uint8_t *w1q, const uint8_t *w1s,
                    const uint8_t *w2q, const uint8_t *w2s, double *g, double *u, double *a,
                    uint8_t *aq, uint8_t *as_, double *o)
{
    double *ab = (double *)malloc(sizeof(double) * (size_t)I);
    for (int32_t i = 0; i < I; ++i) {
        double sg = 0.0, su = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            double xv = mx_value(xq, xs, H, t, h);
            sg += xv * mx_value(w1q, w1s, H, (int64_t)e * 2 * I + i, h);
            su += xv * mx_value(w1q, w1s, H, (int64_t)e * 2 * I + I + i, h);
        }
        g[i] = sg;
        u[i] = su;
        a[i] = silu(sg) * su;
        ab[i] = bf(f32_to_bf16((float)a[i]));
    }
    for (int32_t b = 0; b < I / 32; ++b) as_[b] = mx_block(ab + b * 32, 32, aq + b * 32);
    if (o)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t i = 0; i < I; ++i)
                acc += mx_value(w2q, w2s, I, (int64_t)e * H + h, i) *
                       oracle_e4m3_value(aq[i]) * mx_scale(as_[i / 32]);
            o[h] = acc;
        }
    free(ab);
}

/* Per-slot intermediates of the MXFP8 expert MLP for listed flat slots      */
/* f = t*k + j: g, u, a [n, I] (double), aq [n, I], as_ [n, I/32], o [n, H]. */
void oracle_mx_expert_rows(int32_t H, int32_t I, int32_t k, const uint8_t *xq,
                           const uint8_t *xs, const uint8_t *w1q, const uint8_t *w1s,
                           const uint8_t *w2q, const uint8_t *w2s, const int32_t *idx, int64_t n,
                           const int64_t *slots, double *g, double *u, double *a, uint8_t *aq,
                           uint8_t *as_, double *o)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n; ++q) {
        int64_t f = slots[q];
        mx_slot(H, I, f / k, idx[f], xq, xs, w1q, w1s, w2q, w2s, g + q * I, u + q * I,
                a + q * I, aq + q * I, as_ + q * (I / 32), o + q * H);
    }
}

/* MXFP8 expert forward for a list of tokens (toks == NULL: 0..ntok-1):      */
/*   y[t] = sum_{j ascending} w[t,j] * o(t, idx[t,j])                        */
void oracle_mx_forward(int32_t H, int32_t I, int32_t k, const uint8_t *xq, const uint8_t *xs,
                       const uint8_t *w1q, const uint8_t *w1s, const uint8_t *w2q,
                       const uint8_t *w2s, const int32_t *idx, const double *w, int64_t ntok,
                       const int64_t *toks, double *y)
{
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        uint8_t *aq = (uint8_t *)malloc((size_t)I);
        uint8_t *as_ = (uint8_t *)malloc((size_t)I / 32 + 1);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < ntok; ++q) {
            int64_t t = toks ? toks[q] : q;
            double *yt = y + q * H;
            for (int32_t h = 0; h < H; ++h) yt[h] = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                mx_slot(H, I, t, idx[t * k + j], xq, xs, w1q, w1s, w2q, w2s, g, u, a, aq, as_,
                        o);
                for (int32_t h = 0; h < H; ++h) yt[h] += w[t * k + j] * o[h];
            }
        }
        free(g);
        free(u);
        free(a);
        free(aq);
        free(as_);
        free(o);
    }
}

/* ======================================================================== */
/* MXFP8 backward (page "MegaMoE", "Expert precision": the backward of the   */
/* expert stages and the dW1 / dW2 weight gradients run in MXFP8 too).       */
/* Every GEMM takes its operands in MX form, quantised along its own         */
/* contraction dimension:                                                    */
/*   dA' = DY . W2c^T    DY: dy per token along H;                           */
/*                       W2c: w2[e]^T [I, H] along H (rows e*I + i)          */
/*   dx  = DH . W1c^T    DH: dh per slot along 2I;                           */
/*                       W1c: w1[e]^T [H, 2I] along 2I (rows e*H + h)        */
/*   dW2[e] = DYW_e^T . A_e,  dW1[e] = DH_e^T . XG_e: both operands along    */
/*            the expert's routed rows, in blocks of 32 from its first row   */
/*            (ascending flat slot), the last block padded with zeros.       */
/* Tensors are rounded to the precision the path holds them in before they   */
/* are quantised: dh = bf16(fp32(dg | du)), dyw = bf16(fp32(w * dy)),        */
/* a = bf16(fp32(a)); xg is the bf16 input x.  g, u, a come from the MXFP8   */
/* forward (mx_slot); the SwiGLU backward takes g and u as the forward       */
/* saves them, in h: bf16(fp32(g)), bf16(fp32(u)).  The routing weight's     */
/* gradient is the row-dot dw_j = sum_i dA'_i a_i with the bf16 a.           */
/* ======================================================================== */

/* dA' of one slot (t, e): dAp[i] = sum_h DY[t,h] W2c[e*I+i, h]. */
static void mx_dA(int32_t H, int32_t I, int64_t t, int32_t e, const uint8_t *dyq,
                  const uint8_t *dys, const uint8_t *w2cq, const uint8_t *w2cs, double *dAp)
{
    for (int32_t i = 0; i < I; ++i) {
        double acc = 0.0;
        for (int32_t h = 0; h < H; ++h)
            acc += mx_value(dyq, dys, H, t, h) * mx_value(w2cq, w2cs, H, (int64_t)e * I + i, h);
        dAp[i] = acc;
    }
}

static double bf16_of(double v) { return bf(f32_to_bf16((float)v)); }

/* SwiGLU backward of one element: dg, du from dA = w * dA', g, u. */
static void swiglu_bwd(double dA, double g, double u, double *dg, double *du)
{
    double sg = sigmoid(g);
    *dg = dA * u * sg * (1.0 + g * (1.0 - sg));
    *du = dA * silu(g);
}

/* Backward for a list of tokens: dx [ntok,H], dlogits [ntok,E] (double).    */
/* fwd MX operands: xq/xs [T,H], w1q/w1s [E*2I,H], w2q/w2s [E*H,I];          */
/* backward ones: dyq/dys [T,H], w2cq/w2cs [E*I,H], w1cq/w1cs [E*H,2I].      */
/* w [T,k] routing weights (double); logits [T,E]; Wr [E,H] or NULL.         */
void oracle_mx_backward_tokens(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                               int32_t score, int32_t renorm, double scale, double coeff,
                               double d_aux, const float *Wr, const double *logits,
                               const int32_t *idx, const int32_t *counts, const double *w,
                               const uint8_t *xq, const uint8_t *xs, const uint8_t *w1q,
                               const uint8_t *w1s, const uint8_t *w2q, const uint8_t *w2s,
                               const uint8_t *dyq, const uint8_t *dys, const uint8_t *w2cq,
                               const uint8_t *w2cs, const uint8_t *w1cq, const uint8_t *w1cs,
                               int64_t ntok, const int64_t *toks, double *dx, double *dlogits)
{
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        uint8_t *aq = (uint8_t *)malloc((size_t)I);
        uint8_t *as_ = (uint8_t *)malloc((size_t)I / 32 + 1);
        double *dAp = (double *)malloc(sizeof(double) * (size_t)I);
        double *dh = (double *)malloc(sizeof(double) * 2 * (size_t)I);
        uint8_t *dhq = (uint8_t *)malloc(2 * (size_t)I);
        uint8_t *dhs = (uint8_t *)malloc(2 * (size_t)I / 32 + 1);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        double *dp = (double *)malloc(sizeof(double) * (size_t)E);
        double *dw = (double *)malloc(sizeof(double) * (size_t)k);
        double *wt = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            int64_t t = toks ? toks[n] : n;
            double *dxt = dx + n * H;
            for (int32_t h = 0; h < H; ++h) dxt[h] = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = idx[t * k + j];
                mx_slot(H, I, t, e, xq, xs, w1q, w1s, w2q, w2s, g, u, a, aq, as_, NULL);
                mx_dA(H, I, t, e, dyq, dys, w2cq, w2cs, dAp);
                double acc = 0.0;
                for (int32_t i = 0; i < I; ++i) acc += dAp[i] * bf16_of(a[i]);
                dw[j] = acc;
                for (int32_t i = 0; i < I; ++i) {
                    double dg, du;
                    /* g, u as the forward saved them: h in bf16 */
                    swiglu_bwd(w[t * k + j] * dAp[i], bf16_of(g[i]), bf16_of(u[i]), &dg, &du);
                    dh[i] = bf16_of(dg);
                    dh[I + i] = bf16_of(du);
                }
                for (int32_t b = 0; b < 2 * I / 32; ++b) dhs[b] = mx_block(dh + b * 32, 32, dhq + b * 32);
                for (int32_t h = 0; h < H; ++h) {
                    double s = 0.0;
                    for (int32_t c = 0; c < 2 * I; ++c)
                        s += oracle_e4m3_value(dhq[c]) * mx_scale(dhs[c / 32]) *
                             mx_value(w1cq, w1cs, 2 * I, (int64_t)e * H + h, c);
                    dxt[h] += s;
                }
            }
            router_token_backward(T, H, E, k, score, renorm, scale, coeff, d_aux, Wr,
                                  logits + t * E, idx + t * k, counts, dw, wt, p, dp,
                                  dlogits + n * E, dxt);
        }
        free(g);
        free(u);
        free(a);
        free(aq);
        free(as_);
        free(dAp);
        free(dh);
        free(dhq);
        free(dhs);
        free(p);
        free(dp);
        free(dw);
        free(wt);
    }
}

/* MX value of entry q of a column held as n doubles, quantised in blocks of */
/* 32 from its first entry (the last block padded with zeros).               */
static void mx_column(const double *col, int64_t n, double *out)
{
    double v[32];
    uint8_t c[32];
    for (int64_t b = 0; b < n; b += 32) {
        int64_t m = n - b < 32 ? n - b : 32;
        for (int i = 0; i < 32; ++i) v[i] = i < m ? col[b + i] : 0.0;
        uint8_t s = mx_block(v, 32, c);
        for (int i = 0; i < m; ++i) out[b + i] = oracle_e4m3_value(c[i]) * mx_scale(s);
    }
}

/* Single elements of the MXFP8 weight gradients (the rows of expert e are   */
/* the flat slots f with idx[f] == e, ascending):                            */
/*   which 2: dW2[e, h, i] = sum_r MX(dyw[:, h])_r MX(a[:, i])_r              */
/*   which 1: dW1[e, n, h] = sum_r MX(dh[:, n])_r  MX(xg[:, h])_r             */
/* x, dy raw bf16 [T,H]; w [T,k] double; MX operands as in the backward.     */
void oracle_mx_weight_grad_elements(int64_t T, int32_t H, int32_t I, int32_t k,
                                    const uint16_t *x, const uint16_t *dy, const int32_t *idx,
                                    const double *w, const uint8_t *xq, const uint8_t *xs,
                                    const uint8_t *w1q, const uint8_t *w1s, const uint8_t *dyq,
                                    const uint8_t *dys, const uint8_t *w2cq,
                                    const uint8_t *w2cs, int64_t nel, const int32_t *which,
                                    const int32_t *ee, const int32_t *rr, const int32_t *cc,
                                    double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nel; ++q) {
        int32_t e = ee[q];
        int64_t n = 0;
        for (int64_t f = 0; f < T * k; ++f) n += idx[f] == e;
        double *c1 = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        double *c2 = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        double *m1 = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        double *m2 = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        int64_t r = 0;
        for (int64_t f = 0; f < T * k; ++f) {
            if (idx[f] != e) continue;
            int64_t t = f / k;
            int32_t i = which[q] == 2 ? cc[q] : rr[q] % I;
            /* g_i, u_i of this row from the MXFP8 forward */
            double sg = 0.0, su = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                double xv = mx_value(xq, xs, H, t, h);
                sg += xv * mx_value(w1q, w1s, H, (int64_t)e * 2 * I + i, h);
                su += xv * mx_value(w1q, w1s, H, (int64_t)e * 2 * I + I + i, h);
            }
            if (which[q] == 2) {
                c1[r] = bf16_of(w[f] * bf(dy[t * H + rr[q]]));
                c2[r] = bf16_of(silu(sg) * su);
            } else {
                double dAp = 0.0;
                for (int32_t h = 0; h < H; ++h)
                    dAp += mx_value(dyq, dys, H, t, h) * mx_value(w2cq, w2cs, H, (int64_t)e * I + i, h);
                double dg, du;
                swiglu_bwd(w[f] * dAp, bf16_of(sg), bf16_of(su), &dg, &du);
                c1[r] = bf16_of(rr[q] < I ? dg : du);
                c2[r] = bf(x[t * H + cc[q]]);
            }
            ++r;
        }
        mx_column(c1, n, m1);
        mx_column(c2, n, m2);
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) acc += m1[i] * m2[i];
        out[q] = acc;
        free(c1);
        free(c2);
        free(m1);
        free(m2);
    }
}

/* Whole lines of the MXFP8 weight gradients, each H long:                  */
/*   which[q] == 1: out[q, h] = dW1[ee[q], rr[q], h]                         */
/*                            = sum_r MX(dh[:, n])_r MX(xg[:, h])_r          */
/*   which[q] == 2: out[q, h] = dW2[ee[q], h, rr[q]]                         */
/*                            = sum_r MX(dyw[:, h])_r MX(a[:, i])_r          */
/* with the rows r of expert e (its flat slots, ascending) and the same      */
/* operands and roundings as oracle_mx_weight_grad_elements; every column    */
/* is quantised in blocks of 32 from the expert's first row.  abs_out       */
/* (optional, [nl, H]) receives the sums of the terms' magnitudes,          */
/* sum_r |MX(.)_r MX(.)_r|, the scale of each sum's rounding.               */
void oracle_mx_weight_grad_lines(int64_t T, int32_t H, int32_t I, int32_t k,
                                 const uint16_t *x, const uint16_t *dy, const int32_t *idx,
                                 const double *w, const uint8_t *xq, const uint8_t *xs,
                                 const uint8_t *w1q, const uint8_t *w1s, const uint8_t *dyq,
                                 const uint8_t *dys, const uint8_t *w2cq, const uint8_t *w2cs,
                                 int64_t nl, const int32_t *which, const int32_t *ee,
                                 const int32_t *rr, double *out, double *abs_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nl; ++q) {
        const int32_t e = ee[q];
        const int32_t i = which[q] == 2 ? rr[q] : rr[q] % I;
        int64_t n = 0;
        for (int64_t f = 0; f < T * k; ++f) n += idx[f] == e;
        int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n + 1));
        double *fixed = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        double *mfixed = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        double *col = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        double *mcol = (double *)malloc(sizeof(double) * (size_t)(n + 1));
        int64_t r = 0;
        for (int64_t f = 0; f < T * k; ++f)
            if (idx[f] == e) slot[r++] = f;
        /* the column shared by the whole line: a[:, i] or dh[:, n] */
        for (r = 0; r < n; ++r) {
            const int64_t f = slot[r], t = f / k;
            double sg = 0.0, su = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                double xv = mx_value(xq, xs, H, t, h);
                sg += xv * mx_value(w1q, w1s, H, (int64_t)e * 2 * I + i, h);
                su += xv * mx_value(w1q, w1s, H, (int64_t)e * 2 * I + I + i, h);
            }
            if (which[q] == 2) {
                fixed[r] = bf16_of(silu(sg) * su);
            } else {
                double dAp = 0.0;
                for (int32_t h = 0; h < H; ++h)
                    dAp += mx_value(dyq, dys, H, t, h) *
                           mx_value(w2cq, w2cs, H, (int64_t)e * I + i, h);
                double dg, du;
                swiglu_bwd(w[f] * dAp, bf16_of(sg), bf16_of(su), &dg, &du);
                fixed[r] = bf16_of(rr[q] < I ? dg : du);
            }
        }
        mx_column(fixed, n, mfixed);
        /* the other operand's column h, for every h */
        for (int32_t h = 0; h < H; ++h) {
            for (r = 0; r < n; ++r) {
                const int64_t f = slot[r], t = f / k;
                col[r] = which[q] == 2 ? bf16_of(w[f] * bf(dy[t * H + h])) : bf(x[t * H + h]);
            }
            mx_column(col, n, mcol);
            double acc = 0.0, mag = 0.0;
            for (r = 0; r < n; ++r) {
                acc += mfixed[r] * mcol[r];
                mag += fabs(mfixed[r] * mcol[r]);
            }
            out[q * H + h] = acc;
            if (abs_out) abs_out[q * H + h] = mag;
        }
        free(slot);
        free(fixed);
        free(mfixed);
        free(col);
        free(mcol);
    }
}
