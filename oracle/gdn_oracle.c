/*
 * Test infrastructure, not product code: only tests/, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.
 *
 * Plain fp64 CPU oracle of the gated delta rule, written as the token-by-token
 * recurrence that the chunked form of the MaxText PR "Add context parallelism
 * to the Gated Delta Net (Qwen3-Next / Qwen3.5)" rearranges (section "Why",
 * the affine chunk equations for h_out and o; the page calls the method a
 * "sequential recurrence" in its "Limitation" section).
 *
 * With the state kept K-major, h in R^{K x V} (the page's U is (B,H,K,V); the
 * serving RFC "RFC(qwen35): TP Phase 2", section "Partition Contract", keeps
 * the recurrent state as [H_v, K, V] f32), one token t does
 *
 *     alpha = exp(g_t)
 *     h     <- alpha * h
 *     delta  = beta_t * (v_t - h^T k_t)          (length V)
 *     h     <- h + k_t delta^T
 *     o_t    = h^T q_t                           (length V)
 *
 * which is S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 * o_t = S_t q_t with S = h^T.  No blocking, no reordering, no fast math:
 * exp() is the host libm, every loop runs in the textbook order.
 *
 * Layouts (row-major, contiguous):
 *   batch mode   q,k [B,S,H,K]  v,o [B,S,H,V]  g,beta [B,S,H]  h0,hT [B,H,K,V]
 *   packed mode  q,k [T,H,K]    v,o [T,H,V]    g,beta [T,H]    h0,hT [N,H,K,V]
 *                with sequence n owning tokens cu[n] .. cu[n+1]-1.
 * h0 may be NULL (zero initial state); o and hT may be NULL (not written).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One independent chain (one sequence, one head).  `tok_*` are the strides,
 * in elements, between consecutive tokens of the chain. */
static void run_chain(int S, int K, int V,
                      const double *q, const double *k, const double *v,
                      long tok_qk, long tok_v,
                      const double *g, const double *beta, long tok_gb,
                      double *h, /* K*V: in initial state, out final state */
                      double *o, long tok_o,
                      double *delta /* V scratch */)
{
    for (int t = 0; t < S; ++t) {
        const double *qt = q ? q + (long)t * tok_qk : NULL;
        const double *kt = k + (long)t * tok_qk;
        const double *vt = v + (long)t * tok_v;
        const double alpha = exp(g[(long)t * tok_gb]);
        const double b = beta[(long)t * tok_gb];

        for (int i = 0; i < K; ++i)
            for (int j = 0; j < V; ++j)
                h[(long)i * V + j] *= alpha;

        for (int j = 0; j < V; ++j) {
            double hk = 0.0;
            for (int i = 0; i < K; ++i)
                hk += h[(long)i * V + j] * kt[i];
            delta[j] = b * (vt[j] - hk);
        }

        for (int i = 0; i < K; ++i)
            for (int j = 0; j < V; ++j)
                h[(long)i * V + j] += kt[i] * delta[j];

        if (o) {
            double *ot = o + (long)t * tok_o;
            for (int j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i)
                    acc += h[(long)i * V + j] * qt[i];
                ot[j] = acc;
            }
        }
    }
}

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Batch mode: B sequences of S tokens each, H heads.  Returns 0 on success. */
int gdn_oracle_forward(int B, int S, int H, int K, int V,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       const double *h0, double *o, double *hT, int nthreads)
{
    if (B < 0 || S < 0 || H <= 0 || K <= 0 || V <= 0 || !k || !v || !g || !beta)
        return 1;
    if (o && !q)
        return 1;
    const long KV = (long)K * V;
    const int nchains = B * H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int c = 0; c < nchains; ++c) {
        const int b = c / H, hh = c % H;
        double *h = (double *)malloc(sizeof(double) * (size_t)KV);
        double *delta = (double *)malloc(sizeof(double) * (size_t)V);
        if (!h || !delta) {
            bad = 1;
            free(h);
            free(delta);
            continue;
        }
        if (h0)
            memcpy(h, h0 + (long)c * KV, sizeof(double) * (size_t)KV);
        else
            memset(h, 0, sizeof(double) * (size_t)KV);
        const long tok0 = (long)b * S * H + hh; /* token 0 of this chain, in [B,S,H] units */
        run_chain(S, K, V,
                  q ? q + tok0 * K : NULL, k + tok0 * K, v + tok0 * V,
                  (long)H * K, (long)H * V,
                  g + tok0, beta + tok0, H,
                  h, o ? o + tok0 * V : NULL, (long)H * V, delta);
        if (hT)
            memcpy(hT + (long)c * KV, h, sizeof(double) * (size_t)KV);
        free(h);
        free(delta);
    }
    return bad;
}

/* Packed mode: N sequences laid end to end on one token axis of T = cu[N]
 * tokens; sequence n owns tokens cu[n] .. cu[n+1]-1.  Returns 0 on success. */
int gdn_oracle_forward_packed(int N, const int *cu, int H, int K, int V,
                              const double *q, const double *k, const double *v,
                              const double *g, const double *beta,
                              const double *h0, double *o, double *hT, int nthreads)
{
    if (N < 0 || !cu || H <= 0 || K <= 0 || V <= 0 || !k || !v || !g || !beta)
        return 1;
    if (o && !q)
        return 1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n] || cu[0] != 0)
            return 1;
    const long KV = (long)K * V;
    const int nchains = N * H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int c = 0; c < nchains; ++c) {
        const int n = c / H, hh = c % H;
        double *h = (double *)malloc(sizeof(double) * (size_t)KV);
        double *delta = (double *)malloc(sizeof(double) * (size_t)V);
        if (!h || !delta) {
            bad = 1;
            free(h);
            free(delta);
            continue;
        }
        if (h0)
            memcpy(h, h0 + (long)c * KV, sizeof(double) * (size_t)KV);
        else
            memset(h, 0, sizeof(double) * (size_t)KV);
        const long tok0 = (long)cu[n] * H + hh;
        run_chain(cu[n + 1] - cu[n], K, V,
                  q ? q + tok0 * K : NULL, k + tok0 * K, v + tok0 * V,
                  (long)H * K, (long)H * V,
                  g + tok0, beta + tok0, H,
                  h, o ? o + tok0 * V : NULL, (long)H * V, delta);
        if (hT)
            memcpy(hT + (long)c * KV, h, sizeof(double) * (size_t)KV);
        free(h);
        free(delta);
    }
    return bad;
}

/*
 * Reverse mode.  The gradients of a scalar loss l(o, hT) with respect to every
 * input, given dout = dl/do and dhT = dl/dhT: the vector-Jacobian product of
 * the recurrence above, taken token by token from the last token back.  The
 * pages define no backward pass of their own (the MaxText PR tests one against
 * the recurrence, section "Tests"); this is the chain rule applied to the
 * definition and nothing else.  With hb = alpha h_{t-1} and
 * e = v_t - hb^T k_t (so delta = beta_t e), token t contributes
 *
 *     dq_t    = h_t dout_t                         (o_t = h_t^T q_t)
 *     dh     += q_t dout_t^T
 *     ddelta  = dh^T k_t                           (h_t = hb + k_t delta^T)
 *     dk_t    = dh delta - beta_t hb ddelta
 *     dv_t    = beta_t ddelta
 *     dbeta_t = ddelta . e
 *     dhb     = dh - beta_t k_t ddelta^T
 *     dg_t    = <dhb, hb>                          (hb = exp(g_t) h_{t-1})
 *     dh      = alpha dhb                          (now dl/dh_{t-1})
 *
 * and dh0 is the final dh.  Every state h_0 .. h_S of a chain is kept in
 * memory ((S+1) K V doubles per chain in flight), so this is for test sizes.
 */
static int backward_chain(int S, int K, int V,
                          const double *q, const double *k, const double *v,
                          long tok_qk, long tok_v,
                          const double *g, const double *beta, long tok_gb,
                          const double *h0, const double *dout, const double *dhT,
                          double *dq, double *dk, double *dv, double *dg, double *dbeta,
                          double *dh0)
{
    const long KV = (long)K * V;
    double *hs = (double *)malloc(sizeof(double) * (size_t)(KV * (S + 1)));
    double *hb = (double *)malloc(sizeof(double) * (size_t)KV);
    double *dh = (double *)malloc(sizeof(double) * (size_t)KV);
    double *e = (double *)malloc(sizeof(double) * (size_t)V);
    double *dd = (double *)malloc(sizeof(double) * (size_t)V);
    if (!hs || !hb || !dh || !e || !dd) {
        free(hs); free(hb); free(dh); free(e); free(dd);
        return 1;
    }
    if (h0)
        memcpy(hs, h0, sizeof(double) * (size_t)KV);
    else
        memset(hs, 0, sizeof(double) * (size_t)KV);
    for (int t = 0; t < S; ++t) {
        memcpy(hs + (t + 1) * KV, hs + t * KV, sizeof(double) * (size_t)KV);
        run_chain(1, K, V, NULL, k + (long)t * tok_qk, v + (long)t * tok_v, tok_qk, tok_v,
                  g + (long)t * tok_gb, beta + (long)t * tok_gb, tok_gb,
                  hs + (t + 1) * KV, NULL, 0, e);
    }
    if (dhT)
        memcpy(dh, dhT, sizeof(double) * (size_t)KV);
    else
        memset(dh, 0, sizeof(double) * (size_t)KV);

    for (int t = S - 1; t >= 0; --t) {
        const double *qt = q + (long)t * tok_qk;
        const double *kt = k + (long)t * tok_qk;
        const double *vt = v + (long)t * tok_v;
        const double *dot = dout + (long)t * tok_v;
        const double *hprev = hs + t * KV, *hcur = hs + (t + 1) * KV;
        const double alpha = exp(g[(long)t * tok_gb]);
        const double b = beta[(long)t * tok_gb];
        double *dqt = dq + (long)t * tok_qk, *dkt = dk + (long)t * tok_qk;
        double *dvt = dv + (long)t * tok_v;

        for (int i = 0; i < K; ++i) {
            double acc = 0.0;
            for (int j = 0; j < V; ++j)
                acc += hcur[(long)i * V + j] * dot[j];
            dqt[i] = acc;
        }
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < V; ++j)
                dh[(long)i * V + j] += qt[i] * dot[j];

        for (long x = 0; x < KV; ++x)
            hb[x] = alpha * hprev[x];
        for (int j = 0; j < V; ++j) {
            double pred = 0.0, acc = 0.0;
            for (int i = 0; i < K; ++i) {
                pred += hb[(long)i * V + j] * kt[i];
                acc += dh[(long)i * V + j] * kt[i];
            }
            e[j] = vt[j] - pred;
            dd[j] = acc;
        }
        double db = 0.0;
        for (int j = 0; j < V; ++j) {
            db += dd[j] * e[j];
            dvt[j] = b * dd[j];
        }
        dbeta[(long)t * tok_gb] = db;
        for (int i = 0; i < K; ++i) {
            double acc = 0.0;
            for (int j = 0; j < V; ++j)
                acc += dh[(long)i * V + j] * (b * e[j]) - b * hb[(long)i * V + j] * dd[j];
            dkt[i] = acc;
        }
        double dgt = 0.0;
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < V; ++j) {
                const long x = (long)i * V + j;
                const double dhbx = dh[x] - b * kt[i] * dd[j];
                dgt += dhbx * hb[x];
                dh[x] = alpha * dhbx;
            }
        dg[(long)t * tok_gb] = dgt;
    }
    if (dh0)
        memcpy(dh0, dh, sizeof(double) * (size_t)KV);
    free(hs); free(hb); free(dh); free(e); free(dd);
    return 0;
}

/* Batch-mode backward: layouts as the forward, gradients in the layout of
 * their inputs.  dhT and h0 may be NULL (zero); dh0 may be NULL (not written).
 * Returns 0 on success. */
int gdn_oracle_backward(int B, int S, int H, int K, int V,
                        const double *q, const double *k, const double *v,
                        const double *g, const double *beta, const double *h0,
                        const double *dout, const double *dhT,
                        double *dq, double *dk, double *dv, double *dg, double *dbeta,
                        double *dh0, int nthreads)
{
    if (B < 0 || S < 0 || H <= 0 || K <= 0 || V <= 0 || !q || !k || !v || !g || !beta ||
        !dout || !dq || !dk || !dv || !dg || !dbeta)
        return 1;
    const long KV = (long)K * V;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int c = 0; c < B * H; ++c) {
        const int b = c / H, hh = c % H;
        const long tok0 = (long)b * S * H + hh;
        if (backward_chain(S, K, V, q + tok0 * K, k + tok0 * K, v + tok0 * V,
                           (long)H * K, (long)H * V, g + tok0, beta + tok0, H,
                           h0 ? h0 + c * KV : NULL, dout + tok0 * V, dhT ? dhT + c * KV : NULL,
                           dq + tok0 * K, dk + tok0 * K, dv + tok0 * V, dg + tok0, dbeta + tok0,
                           dh0 ? dh0 + c * KV : NULL))
            bad = 1;
    }
    return bad;
}

/* Packed-mode backward: sequence n owns tokens cu[n] .. cu[n+1]-1. */
int gdn_oracle_backward_packed(int N, const int *cu, int H, int K, int V,
                               const double *q, const double *k, const double *v,
                               const double *g, const double *beta, const double *h0,
                               const double *dout, const double *dhT,
                               double *dq, double *dk, double *dv, double *dg, double *dbeta,
                               double *dh0, int nthreads)
{
    if (N < 0 || !cu || H <= 0 || K <= 0 || V <= 0 || !q || !k || !v || !g || !beta ||
        !dout || !dq || !dk || !dv || !dg || !dbeta)
        return 1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n] || cu[0] != 0)
            return 1;
    const long KV = (long)K * V;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int c = 0; c < N * H; ++c) {
        const int n = c / H, hh = c % H;
        const long tok0 = (long)cu[n] * H + hh;
        if (backward_chain(cu[n + 1] - cu[n], K, V, q + tok0 * K, k + tok0 * K, v + tok0 * V,
                           (long)H * K, (long)H * V, g + tok0, beta + tok0, H,
                           h0 ? h0 + c * KV : NULL, dout + tok0 * V, dhT ? dhT + c * KV : NULL,
                           dq + tok0 * K, dk + tok0 * K, dv + tok0 * V, dg + tok0, dbeta + tok0,
                           dh0 ? dh0 + c * KV : NULL))
            bad = 1;
    }
    return bad;
}
