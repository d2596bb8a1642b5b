/*
 * oracle.c — the reference semantics of causal linear-attention sequence
 * mixing with a fixed d_k x d_v state per head, written as the plain
 * token-by-token recurrence in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker for the HIP path.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header or constant with the HIP library and it
 * never sees a value that the HIP library produced.
 *
 * Sources (page titles as published):
 *   [LAV]  "Linear Attention, Visualized" (snowchord.com; wpnews.pro copy)
 *   [BA]   "Beyond attention" (learning.iampt.xyz)
 *   [ASF]  "All sorts of famous Attention Layers" (harsh-ps-2003 blog)
 *
 * What is computed, per (batch b, head h), independently, for t = 1..T, with
 * S_0 given (zero when no initial state is passed):
 *
 *   a_t  = exp(g_t)          log-gate g; scalar per token, or one value per
 *                            key channel (row of S).  No gate: a_t = 1.
 *   S'   = a_t * S_{t-1}     scalar gate: the whole state shrinks
 *                            ([LAV] "Mamba-2: input-dependent scalar decay",
 *                             [BA] "Three ways to update the state": Decay)
 *        = Diag(a_t) S_{t-1} channel gate: row i (key channel i) shrinks by
 *                            a_t[i] ([LAV] "Gated Linear Attention (GLA)")
 *   add  : S_t = S' + k_t^T v_t
 *                            ([LAV] "Naive linear attention"; [BA] "Add")
 *   delta: vhat = k_t S' ; u = beta_t (v_t - vhat) ; S_t = S' + k_t^T u
 *                            ([LAV] "DeltaNet: correcting memory collisions",
 *                             recurrent form with the scaled correction u_t;
 *                             [ASF] "DeltaNet": read v_old at k, write the
 *                             beta-scaled difference).  With a gate this is
 *                             Gated DeltaNet ([LAV] "Gated DeltaNet (GDN)")
 *                             and, for a channel gate, Kimi Delta Attention,
 *                             which decays first and then applies the delta
 *                             correction ([LAV] "Kimi Delta Attention (KDA)").
 *   o_t  = q_t S_t           read-out after the token's own write, so the
 *                            output includes token t ([LAV] "Naive linear
 *                            attention", inclusive causal mask).
 *
 * Row-vector convention as in [LAV] "Self-attention recap": q_t, k_t are
 * 1 x d_k, v_t is 1 x d_v, S is d_k x d_v, stored row-major (S[i*dv + j]).
 * No query scaling, no normaliser: neither appears in the read-out on [LAV].
 *
 * oracle_recurrence_bwd differentiates the same recurrence in reverse (the
 * gradients of a training step); oracle_deltaproduct (and its backward) and
 * oracle_normalized are the Gated DeltaProduct and normalised variants, each
 * described where defined.
 *
 * Arithmetic: IEEE fp64, plain loops, fixed order per head.  OpenMP
 * parallelises over independent (b, h) pairs only, so the result does not
 * depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_RULE_ADD = 0, ORACLE_RULE_DELTA = 1 };
enum { ORACLE_GATE_NONE = 0, ORACLE_GATE_SCALAR = 1, ORACLE_GATE_CHANNEL = 2 };

/* One token of one head, in place on S (dk x dv).  u is dv doubles of scratch. */
static void token_update(int dk, int dv, int rule, int gate,
                         const double *q, const double *k, const double *v,
                         const double *g, double beta,
                         double *S, double *o, double *u)
{
    int i, j;
    /* decay the previous state: S' = a S (scalar) or Diag(a) S (channel) */
    if (gate == ORACLE_GATE_SCALAR) {
        double a = exp(g[0]);
        for (i = 0; i < dk * dv; ++i) S[i] *= a;
    } else if (gate == ORACLE_GATE_CHANNEL) {
        for (i = 0; i < dk; ++i) {
            double a = exp(g[i]);
            for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
        }
    }
    /* the value written at k_t: v itself (add) or beta (v - k S') (delta) */
    if (rule == ORACLE_RULE_DELTA) {
        for (j = 0; j < dv; ++j) {
            double vhat = 0.0;
            for (i = 0; i < dk; ++i) vhat += k[i] * S[(size_t)i * dv + j];
            u[j] = beta * (v[j] - vhat);
        }
    } else {
        for (j = 0; j < dv; ++j) u[j] = v[j];
    }
    /* rank-one write k^T u */
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * u[j];
    /* read-out o = q S (after the write) */
    for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
        o[j] = acc;
    }
}

static int check_args(int64_t B, int64_t H, int64_t T, int dk, int dv, int rule, int gate,
                      const void *q, const void *k, const void *v, const void *g,
                      const void *beta, const void *o)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 2;
    if (rule != ORACLE_RULE_ADD && rule != ORACLE_RULE_DELTA) return 3;
    if (gate < ORACLE_GATE_NONE || gate > ORACLE_GATE_CHANNEL) return 3;
    if (B * H * T > 0 && (!q || !k || !v || !o)) return 1;
    if (gate != ORACLE_GATE_NONE && B * H * T > 0 && !g) return 1;
    if (rule == ORACLE_RULE_DELTA && B * H * T > 0 && !beta) return 1;
    return 0;
}

/*
 * Full forward over a sequence.  Layouts (row-major, contiguous):
 *   q, k  [B,H,T,dk]   v, o  [B,H,T,dv]
 *   g     [B,H,T] (scalar gate) | [B,H,T,dk] (channel gate) | NULL (no gate)
 *   beta  [B,H,T] (delta rule)  | NULL (add rule)
 *   s0    [B,H,dk,dv] or NULL (zero initial state)
 *   s_final [B,H,dk,dv] or NULL
 * Returns 0 on success, nonzero on invalid arguments (nothing written).
 */
int oracle_recurrence(int64_t B, int64_t H, int64_t T, int dk, int dv, int rule, int gate,
                      const double *q, const double *k, const double *v,
                      const double *g, const double *beta, const double *s0,
                      double *o, double *s_final, int nthreads)
{
    int rc = check_args(B, H, T, dk, dv, rule, gate, q, k, v, g, beta, o);
    if (rc) return rc;
    int64_t nheads = B * H;
    size_t ss = (size_t)dk * dv;
    int64_t bh;
    int failed = 0;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : failed)
#else
    (void)nthreads;
#endif
    for (bh = 0; bh < nheads; ++bh) {
        double *S = (double *)malloc(ss * sizeof(double));
        double *u = (double *)malloc((size_t)dv * sizeof(double));
        if (!S || !u) { free(S); free(u); failed |= 1; continue; }
        if (s0) memcpy(S, s0 + (size_t)bh * ss, ss * sizeof(double));
        else memset(S, 0, ss * sizeof(double));
        int64_t t;
        for (t = 0; t < T; ++t) {
            size_t tok = (size_t)bh * (size_t)T + (size_t)t;
            const double *gt = NULL;
            if (gate == ORACLE_GATE_SCALAR) gt = g + tok;
            else if (gate == ORACLE_GATE_CHANNEL) gt = g + tok * dk;
            double bt = (rule == ORACLE_RULE_DELTA) ? beta[tok] : 0.0;
            token_update(dk, dv, rule, gate, q + tok * dk, k + tok * dk, v + tok * dv,
                         gt, bt, S, o + tok * dv, u);
        }
        if (s_final) memcpy(s_final + (size_t)bh * ss, S, ss * sizeof(double));
        free(S);
        free(u);
    }
    return failed ? 6 : 0;
}

/*
 * One decode step: the same recurrence with one token per (sequence n, head h),
 * applied to the state in place.  Layouts: q, k [N,H,dk]; v, o [N,H,dv];
 * g [N,H] | [N,H,dk] | NULL; beta [N,H] | NULL; state [N,H,dk,dv] (in/out).
 */
int oracle_decode_step(int64_t N, int64_t H, int dk, int dv, int rule, int gate,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta, double *state,
                       double *o, int nthreads)
{
    int rc = check_args(N, H, 1, dk, dv, rule, gate, q, k, v, g, beta, o);
    if (rc) return rc;
    if (N * H > 0 && !state) return 1;
    return oracle_recurrence(N, H, 1, dk, dv, rule, gate, q, k, v, g, beta, state, o, state,
                             nthreads);
}

/*
 * Gated DeltaProduct ([LAV] "Gated Delta Product (GDP)"): each token applies
 * an ordered product of n_h generalized Householder transitions, each with its
 * own key, value and correction gate, after decaying the previous state once:
 *
 *   S = a_t S_{t-1}                                  (scalar gate; none: a_t = 1)
 *   for j = 1..n_h:  S = S + k_{t,j}^T beta_{t,j} (v_{t,j} - k_{t,j} S)
 *   S_t = S ;  o_t = q_t S_t                         (query after the last substep)
 *
 * Layouts: q [B,H,T,dk]; k [B,H,T,nh,dk]; v [B,H,T,nh,dv]; beta [B,H,T,nh];
 * g [B,H,T] or NULL; s0, s_final [B,H,dk,dv]; o [B,H,T,dv].  Written as its own
 * loop (not through token_update), so that checking n_h = 1 against the delta
 * rule above compares two separate codes.
 */
int oracle_deltaproduct(int64_t B, int64_t H, int64_t T, int nh, int dk, int dv, int gate,
                        const double *q, const double *k, const double *v,
                        const double *g, const double *beta, const double *s0,
                        double *o, double *s_final, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || nh <= 0 || dk <= 0 || dv <= 0) return 2;
    if (gate != ORACLE_GATE_NONE && gate != ORACLE_GATE_SCALAR) return 3;
    if (B * H * T > 0 && (!q || !k || !v || !beta || !o)) return 1;
    if (gate == ORACLE_GATE_SCALAR && B * H * T > 0 && !g) return 1;
    int64_t nheads = B * H;
    size_t ss = (size_t)dk * dv;
    int64_t bh;
    int failed = 0;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : failed)
#else
    (void)nthreads;
#endif
    for (bh = 0; bh < nheads; ++bh) {
        double *S = (double *)malloc(ss * sizeof(double));
        double *w = (double *)malloc((size_t)dv * sizeof(double));
        if (!S || !w) { free(S); free(w); failed |= 1; continue; }
        if (s0 != NULL) memcpy(S, s0 + (size_t)bh * ss, ss * sizeof(double));
        else memset(S, 0, ss * sizeof(double));
        int64_t t;
        int i, j, c;
        for (t = 0; t < T; ++t) {
            size_t tok = (size_t)bh * (size_t)T + (size_t)t;
            if (gate == ORACLE_GATE_SCALAR) {
                double a = exp(g[tok]);
                for (i = 0; i < dk * dv; ++i) S[i] *= a;
            }
            for (j = 0; j < nh; ++j) {
                const double *kj = k + (tok * nh + j) * dk;
                const double *vj = v + (tok * nh + j) * dv;
                double bj = beta[tok * nh + j];
                /* w = beta (v - k S): the correction written at k */
                for (c = 0; c < dv; ++c) {
                    double pred = 0.0;
                    for (i = 0; i < dk; ++i) pred += kj[i] * S[(size_t)i * dv + c];
                    w[c] = bj * (vj[c] - pred);
                }
                for (i = 0; i < dk; ++i)
                    for (c = 0; c < dv; ++c) S[(size_t)i * dv + c] += kj[i] * w[c];
            }
            const double *qt = q + tok * dk;
            for (c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (i = 0; i < dk; ++i) acc += qt[i] * S[(size_t)i * dv + c];
                o[tok * dv + c] = acc;
            }
        }
        if (s_final) memcpy(s_final + (size_t)bh * ss, S, ss * sizeof(double));
        free(S);
        free(w);
    }
    return failed ? 6 : 0;
}

/*
 * Normalised linear attention ("All sorts of famous Attention Layers",
 * "Linear Magic" and the normaliser of the linear-attention layer there): the
 * add rule with a second state z_t, the (decayed) running sum of the keys, and
 * the read-out divided by q_t . z_t:
 *
 *   a_t = exp(g_t) (scalar gate), a vector (channel gate: row r of S and
 *   entry r of z decay by a_t[r]) or 1;  S_t = a_t S_{t-1} + k_t^T v_t;
 *   z_t = a_t z_{t-1} + k_t;  o_t = (q_t S_t) / (q_t . z_t)
 *
 * q, k are the feature-mapped queries and keys (positive for elu + 1, so the
 * denominator is positive).  Layouts: q, k [B,H,T,dk]; v, o [B,H,T,dv];
 * g [B,H,T] | [B,H,T,dk] | NULL; s0, s_final [B,H,dk,dv]; z0, z_final [B,H,dk].
 */
int oracle_normalized(int64_t B, int64_t H, int64_t T, int dk, int dv, int gate,
                      const double *q, const double *k, const double *v, const double *g,
                      const double *s0, const double *z0, double *o, double *s_final,
                      double *z_final, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 2;
    if (gate < ORACLE_GATE_NONE || gate > ORACLE_GATE_CHANNEL) return 3;
    if (B * H * T > 0 && (!q || !k || !v || !o)) return 1;
    if (gate != ORACLE_GATE_NONE && B * H * T > 0 && !g) return 1;
    int64_t nheads = B * H;
    size_t ss = (size_t)dk * dv;
    int64_t bh;
    int failed = 0;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : failed)
#else
    (void)nthreads;
#endif
    for (bh = 0; bh < nheads; ++bh) {
        double *S = (double *)malloc(ss * sizeof(double));
        double *z = (double *)malloc((size_t)dk * sizeof(double));
        if (!S || !z) { free(S); free(z); failed |= 1; continue; }
        if (s0 != 0) memcpy(S, s0 + (size_t)bh * ss, ss * sizeof(double));
        else memset(S, 0, ss * sizeof(double));
        if (z0 != NULL) memcpy(z, z0 + (size_t)bh * dk, (size_t)dk * sizeof(double));
        else memset(z, 0, (size_t)dk * sizeof(double));
        int64_t t;
        int r, c;
        for (t = 0; t < T; ++t) {
            size_t tok = (size_t)bh * (size_t)T + (size_t)t;
            const double *qt = q + tok * dk, *kt = k + tok * dk, *vt = v + tok * dv;
            for (r = 0; r < dk; ++r) {
                double a = gate == ORACLE_GATE_SCALAR    ? exp(g[tok])
                         : gate == ORACLE_GATE_CHANNEL ? exp(g[tok * dk + r]) : 1.0;
                z[r] = a * z[r] + kt[r];
                for (c = 0; c < dv; ++c) S[(size_t)r * dv + c] = a * S[(size_t)r * dv + c] + kt[r] * vt[c];
            }
            double den = 0.0;
            for (r = 0; r < dk; ++r) den += qt[r] * z[r];
            for (c = 0; c < dv; ++c) {
                double num = 0.0;
                for (r = 0; r < dk; ++r) num += qt[r] * S[(size_t)r * dv + c];
                o[tok * dv + c] = num / den;
            }
        }
        if (s_final) memcpy(s_final + (size_t)bh * ss, S, ss * sizeof(double));
        if (z_final) memcpy(z_final + (size_t)bh * dk, z, (size_t)dk * sizeof(double));
        free(S);
        free(z);
    }
    return failed ? 6 : 0;
}

/*
 * Backward pass of the token recurrence above: the gradients a training step
 * needs ([LAV] "Optional: Linear attention as an RNN" and "Update the state":
 * autograd of the recurrent form keeps every state for the backward pass, the
 * chunk form one per chunk; [BA] "Chunkwise parallel training").
 * Given the gradient of a loss with respect to every output o_t (do) and to the
 * final state S_T (dsT, NULL for zero), it returns the gradients with respect
 * to q, k, v, g, beta and s0, by reverse-mode differentiation of each step of
 * token_update, newest token first:
 *
 *   H      gradient w.r.t. S_t from everything after the read-out of token t
 *          (starts as dsT); the read-out adds q_t^T do_t:  Ht = H + q_t^T do_t
 *   dq_t   = do_t S_t^T
 *   write  S_t = S' + k_t^T u :   du = k_t Ht,  dk_t += Ht u^T,  dS' = Ht
 *   delta  u = beta (v - k S') :  dbeta_t = du . (v - vhat),  dv_t = beta du,
 *          dvhat = -beta du,  dk_t += S' dvhat^T,  dS' += k_t^T dvhat
 *   add    u = v :                dv_t = du
 *   decay  S' = a S_{t-1}, a = exp(g_t):  dg_t = <dS', S'>  (channel gate: one
 *          inner product per row), and the gradient passed to S_{t-1} is a dS'
 *          (row-wise for the channel gate).
 *   ds0    = the gradient left after the first token.
 *
 * States are recomputed rather than stored: the forward keeps S at the start of
 * every segment of SEG tokens, and the backward replays one segment at a time
 * with the same arithmetic (so the replayed states are bit-identical).
 * Layouts as oracle_recurrence; do, dv [B,H,T,dv]; dq, dk [B,H,T,dk];
 * dg like g (NULL when there is no gate); dbeta like beta (NULL for the add
 * rule); ds0 [B,H,dk,dv] or NULL.
 */
enum { ORACLE_BWD_SEG = 64 };

int oracle_recurrence_bwd(int64_t B, int64_t H, int64_t T, int dk, int dv, int rule, int gate,
                          const double *q, const double *k, const double *v,
                          const double *g, const double *beta, const double *s0,
                          const double *dout, const double *dsT,
                          double *dq, double *dk_out, double *dv_out, double *dg,
                          double *dbeta, double *ds0, int nthreads)
{
    int rc = check_args(B, H, T, dk, dv, rule, gate, q, k, v, g, beta, dout);
    if (rc) return rc;
    if (B * H * T > 0 && (!dq || !dk_out || !dv_out)) return 1;
    if (gate != ORACLE_GATE_NONE && B * H * T > 0 && !dg) return 1;
    if (rule == ORACLE_RULE_DELTA && B * H * T > 0 && !dbeta) return 1;
    int64_t nheads = B * H;
    size_t ss = (size_t)dk * dv;
    int64_t nseg = (T + ORACLE_BWD_SEG - 1) / ORACLE_BWD_SEG;
    int64_t bh;
    int failed = 0;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : failed)
#else
    (void)nthreads;
#endif
    for (bh = 0; bh < nheads; ++bh) {
        /* segment start states, the decayed states S' of one segment, the
         * running gradient and small vectors */
        double *ck = (double *)malloc((size_t)(nseg + 1) * ss * sizeof(double));
        double *Sd = (double *)malloc((size_t)ORACLE_BWD_SEG * ss * sizeof(double));
        double *Hg = (double *)malloc(ss * sizeof(double));
        double *St = (double *)malloc(ss * sizeof(double));
        double *u = (double *)malloc((size_t)dv * sizeof(double));
        double *vh = (double *)malloc((size_t)dv * sizeof(double));
        double *du = (double *)malloc((size_t)dv * sizeof(double));
        double *ot = (double *)malloc((size_t)dv * sizeof(double));
        if (!ck || !Sd || !Hg || !St || !u || !vh || !du || !ot) {
            free(ck); free(Sd); free(Hg); free(St); free(u); free(vh); free(du); free(ot);
            failed |= 1;
            continue;
        }
        int i, j;
        int64_t t, sg;
        /* forward: keep the state at the start of every segment */
        if (s0 == NULL) memset(St, 0, ss * sizeof(double));
        else memcpy(St, s0 + (size_t)bh * ss, ss * sizeof(double));
        for (t = 0; t < T; ++t) {
            if (t % ORACLE_BWD_SEG == 0) memcpy(ck + (size_t)(t / ORACLE_BWD_SEG) * ss, St, ss * sizeof(double));
            size_t tok = (size_t)bh * (size_t)T + (size_t)t;
            const double *gt = gate == ORACLE_GATE_SCALAR ? g + tok : gate == ORACLE_GATE_CHANNEL ? g + tok * dk : NULL;
            token_update(dk, dv, rule, gate, q + tok * dk, k + tok * dk, v + tok * dv, gt,
                         rule == ORACLE_RULE_DELTA ? beta[tok] : 0.0, St, ot, u);
        }
        /* backward */
        if (dsT) memcpy(Hg, dsT + (size_t)bh * ss, ss * sizeof(double));
        else memset(Hg, 0, ss * sizeof(double));
        for (sg = nseg - 1; sg >= 0; --sg) {
            int64_t ta = sg * ORACLE_BWD_SEG;
            int64_t tb = ta + ORACLE_BWD_SEG < T ? ta + ORACLE_BWD_SEG : T;
            /* replay the segment, keeping Sd[t - ta] = S' of token t (the decayed S_{t-1}) */
            memcpy(St, ck + (size_t)sg * ss, ss * sizeof(double));
            for (t = ta; t < tb; ++t) {
                size_t tok = (size_t)bh * (size_t)T + (size_t)t;
                const double *gt = gate == ORACLE_GATE_SCALAR ? g + tok : gate == ORACLE_GATE_CHANNEL ? g + tok * dk : NULL;
                double *sd = Sd + (size_t)(t - ta) * ss;
                for (i = 0; i < dk; ++i) {
                    double a = gate == ORACLE_GATE_SCALAR ? exp(gt[0]) : gate == ORACLE_GATE_CHANNEL ? exp(gt[i]) : 1.0;
                    for (j = 0; j < dv; ++j) sd[(size_t)i * dv + j] = a * St[(size_t)i * dv + j];
                }
                token_update(dk, dv, rule, gate, q + tok * dk, k + tok * dk, v + tok * dv, gt,
                             rule == ORACLE_RULE_DELTA ? beta[tok] : 0.0, St, ot, u);
            }
            for (t = tb - 1; t >= ta; --t) {
                size_t tok = (size_t)bh * (size_t)T + (size_t)t;
                const double *qt = q + tok * dk, *kt = k + tok * dk, *vt = v + tok * dv;
                const double *dot = dout + tok * dv;
                const double *sd = Sd + (size_t)(t - ta) * ss;
                double bt = 0.0;
                if (rule == ORACLE_RULE_DELTA) bt = beta[tok];
                /* vhat and u of this token, and S_t = S' + k^T u */
                for (j = 0; j < dv; ++j) {
                    double p = 0.0;
                    for (i = 0; i < dk; ++i) p += kt[i] * sd[(size_t)i * dv + j];
                    vh[j] = p;
                    u[j] = rule == ORACLE_RULE_DELTA ? bt * (vt[j] - p) : vt[j];
                }
                for (i = 0; i < dk; ++i)
                    for (j = 0; j < dv; ++j) St[(size_t)i * dv + j] = sd[(size_t)i * dv + j] + kt[i] * u[j];
                /* read-out o_t = q_t S_t */
                for (i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dv; ++j) acc += dot[j] * St[(size_t)i * dv + j];
                    dq[tok * dk + i] = acc;
                }
                for (i = 0; i < dk; ++i)
                    for (j = 0; j < dv; ++j) Hg[(size_t)i * dv + j] += qt[i] * dot[j];
                /* write S_t = S' + k^T u */
                for (j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dk; ++i) acc += kt[i] * Hg[(size_t)i * dv + j];
                    du[j] = acc;
                }
                for (i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dv; ++j) acc += Hg[(size_t)i * dv + j] * u[j];
                    dk_out[tok * dk + i] = acc;
                }
                if (rule == ORACLE_RULE_DELTA) {
                    double db = 0.0;
                    for (j = 0; j < dv; ++j) db += du[j] * (vt[j] - vh[j]);
                    dbeta[tok] = db;
                    for (j = 0; j < dv; ++j) dv_out[tok * dv + j] = bt * du[j];
                    /* dvhat = -beta du, into k and into S' */
                    for (i = 0; i < dk; ++i) {
                        double acc = 0.0;
                        for (j = 0; j < dv; ++j) acc += sd[(size_t)i * dv + j] * (-bt * du[j]);
                        dk_out[tok * dk + i] += acc;
                    }
                    for (i = 0; i < dk; ++i)
                        for (j = 0; j < dv; ++j) Hg[(size_t)i * dv + j] += kt[i] * (-bt * du[j]);
                } else {
                    for (j = 0; j < dv; ++j) dv_out[tok * dv + j] = du[j];
                }
                /* decay S' = a S_{t-1}; Hg now holds dS' */
                if (gate == ORACLE_GATE_SCALAR) {
                    double acc = 0.0, a = exp(g[tok]);
                    for (i = 0; i < dk * dv; ++i) acc += Hg[i] * sd[i];
                    dg[tok] = acc;
                    for (i = 0; i < dk * dv; ++i) Hg[i] *= a;
                } else if (gate == ORACLE_GATE_CHANNEL) {
                    for (i = 0; i < dk; ++i) {
                        double acc = 0.0, a = exp(g[tok * dk + i]);
                        for (j = 0; j < dv; ++j) acc += Hg[(size_t)i * dv + j] * sd[(size_t)i * dv + j];
                        dg[tok * dk + i] = acc;
                        for (j = 0; j < dv; ++j) Hg[(size_t)i * dv + j] *= a;
                    }
                }
            }
        }
        if (ds0) memcpy(ds0 + (size_t)bh * ss, Hg, ss * sizeof(double));
        free(ck); free(Sd); free(Hg); free(St); free(u); free(vh); free(du); free(ot);
    }
    return failed ? 6 : 0;
}

/*
 * Backward pass of Gated DeltaProduct (oracle_deltaproduct above): the
 * gradients of sum(dout . o) + sum(dsT . S_T) with respect to q, k, v, g,
 * beta and s0.  Per token, newest first: the read-out adds q_t^T dout_t to the
 * running gradient H and gives dq_t = dout_t S_t^T; the substeps are undone
 * last first, each exactly as the delta step in oracle_recurrence_bwd (without
 * a decay of its own); then the token's decay, a_t = exp(g_t) applied once
 * before the first substep, gives dg_t = <H, a_t S_{t-1}> and H <- a_t H.
 * States are recomputed per segment of SEG tokens from checkpoints, and each
 * token's substep states from the state before the token.  Layouts as
 * oracle_deltaproduct; dq [B,H,T,dk], dk [B,H,T,nh,dk], dv [B,H,T,nh,dv],
 * dg [B,H,T] or NULL (no gate), dbeta [B,H,T,nh], ds0 [B,H,dk,dv] or NULL.
 */
int oracle_deltaproduct_bwd(int64_t B, int64_t H, int64_t T, int nh, int dk, int dv, int gate,
                            const double *q, const double *k, const double *v,
                            const double *g, const double *beta, const double *s0,
                            const double *dout, const double *dsT,
                            double *dq, double *dk_out, double *dv_out, double *dg,
                            double *dbeta, double *ds0, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || nh <= 0 || dk <= 0 || dv <= 0) return 2;
    if (gate != ORACLE_GATE_NONE && gate != ORACLE_GATE_SCALAR) return 3;
    if (B * H * T > 0 && (!q || !k || !v || !beta || !dout || !dq || !dk_out || !dv_out || !dbeta)) return 1;
    if (gate == ORACLE_GATE_SCALAR && B * H * T > 0 && (!g || !dg)) return 1;
    int64_t nheads = B * H;
    size_t ss = (size_t)dk * dv;
    int64_t nseg = (T + ORACLE_BWD_SEG - 1) / ORACLE_BWD_SEG;
    int64_t bh;
    int failed = 0;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : failed)
#else
    (void)nthreads;
#endif
    for (bh = 0; bh < nheads; ++bh) {
        /* checkpoints, the state before each token of a segment, the substep
         * states of one token, the running gradient, small vectors */
        double *ck = (double *)malloc((size_t)(nseg + 1) * ss * sizeof(double));
        double *Sp = (double *)malloc((size_t)ORACLE_BWD_SEG * ss * sizeof(double));
        double *Sj = (double *)malloc((size_t)(nh + 1) * ss * sizeof(double));
        double *Hg = (double *)malloc(ss * sizeof(double));
        double *St = (double *)malloc(ss * sizeof(double));
        double *w = (double *)malloc((size_t)dv * sizeof(double));
        double *vh = (double *)malloc((size_t)dv * sizeof(double));
        double *du = (double *)malloc((size_t)dv * sizeof(double));
        if (!ck || !Sp || !Sj || !Hg || !St || !w || !vh || !du) {
            free(ck); free(Sp); free(Sj); free(Hg); free(St); free(w); free(vh); free(du);
            failed |= 1;
            continue;
        }
        int64_t t, sg;
        int i, j, c;
        /* one token forward from St (in place), keeping its substep states in Sj:
         * Sj[0] = a S_{t-1}, Sj[j+1] after substep j */
#define GDP_TOKEN_FWD(tok_)                                                                    \
        do {                                                                                   \
            double a_ = gate == ORACLE_GATE_SCALAR ? exp(g[tok_]) : 1.0;                      \
            for (i = 0; i < dk * dv; ++i) Sj[i] = a_ * St[i];                                  \
            for (j = 0; nh > j; ++j) {                                                         \
                const double *kj = k + ((tok_) * nh + j) * dk;                                 \
                const double *vj = v + ((tok_) * nh + j) * dv;                                 \
                double bj = beta[(tok_) * nh + j];                                             \
                const double *Sa = Sj + (size_t)j * ss;                                        \
                double *Sb = Sj + (size_t)(j + 1) * ss;                                        \
                for (c = 0; c < dv; ++c) {                                                     \
                    double p_ = 0.0;                                                           \
                    for (i = 0; i < dk; ++i) p_ += kj[i] * Sa[(size_t)i * dv + c];             \
                    w[c] = bj * (vj[c] - p_);                                                  \
                }                                                                              \
                for (i = 0; i < dk; ++i)                                                       \
                    for (c = 0; c < dv; ++c) Sb[(size_t)i * dv + c] = Sa[(size_t)i * dv + c] + kj[i] * w[c]; \
            }                                                                                  \
            memcpy(St, Sj + (size_t)nh * ss, ss * sizeof(double));                              \
        } while (0)
        if (NULL != s0) memcpy(St, s0 + (size_t)bh * ss, ss * sizeof(double));
        else memset(St, 0, ss * sizeof(double));
        for (t = 0; t < T; ++t) {
            size_t tok = (size_t)bh * (size_t)T + (size_t)t;
            if (t % ORACLE_BWD_SEG == 0) memcpy(ck + (size_t)(t / ORACLE_BWD_SEG) * ss, St, ss * sizeof(double));
            GDP_TOKEN_FWD(tok);
        }
        if (dsT != NULL) memcpy(Hg, dsT + (size_t)bh * ss, ss * sizeof(double));
        else memset(Hg, 0, ss * sizeof(double));
        for (sg = nseg - 1; sg >= 0; --sg) {
            int64_t ta = sg * ORACLE_BWD_SEG;
            int64_t tb = ta + ORACLE_BWD_SEG < T ? ta + ORACLE_BWD_SEG : T;
            memcpy(St, ck + (size_t)sg * ss, ss * sizeof(double));
            for (t = ta; t < tb; ++t) {
                size_t tok = (size_t)bh * (size_t)T + (size_t)t;
                memcpy(Sp + (size_t)(t - ta) * ss, St, ss * sizeof(double));
                GDP_TOKEN_FWD(tok);
            }
            for (t = tb - 1; t >= ta; --t) {
                size_t tok = (size_t)bh * (size_t)T + (size_t)t;
                memcpy(St, Sp + (size_t)(t - ta) * ss, ss * sizeof(double));
                GDP_TOKEN_FWD(tok);                   /* Sj now holds this token's states */
                const double *qt = q + tok * dk, *dot = dout + tok * dv;
                const double *Sl = Sj + (size_t)nh * ss;
                for (i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (c = 0; c < dv; ++c) acc += dot[c] * Sl[(size_t)i * dv + c];
                    dq[tok * dk + i] = acc;
                }
                for (i = 0; i < dk; ++i)
                    for (c = 0; c < dv; ++c) Hg[(size_t)i * dv + c] += qt[i] * dot[c];
                for (j = nh - 1; j >= 0; --j) {
                    const double *kj = k + (j + tok * nh) * dk;
                    const double *vj = v + (j + tok * nh) * dv;
                    double bj = beta[j + tok * nh];
                    const double *Sa = Sj + (size_t)j * ss;
                    double *dkj = dk_out + (tok * nh + j) * dk;
                    for (c = 0; c < dv; ++c) {
                        double p_ = 0.0, d_ = 0.0;
                        for (i = 0; i < dk; ++i) {
                            p_ += kj[i] * Sa[(size_t)i * dv + c];
                            d_ += kj[i] * Hg[(size_t)i * dv + c];
                        }
                        vh[c] = p_;
                        w[c] = bj * (vj[c] - p_);
                        du[c] = d_;
                    }
                    /* write S_{j+1} = S_j + k^T w */
                    for (i = 0; i < dk; ++i) {
                        double acc = 0.0;
                        for (c = 0; c < dv; ++c) acc += Hg[(size_t)i * dv + c] * w[c];
                        dkj[i] = acc;
                    }
                    double db = 0.0;
                    for (c = 0; c < dv; ++c) db += du[c] * (vj[c] - vh[c]);
                    dbeta[tok * nh + j] = db;
                    for (c = 0; c < dv; ++c) dv_out[(tok * nh + j) * dv + c] = bj * du[c];
                    /* the prediction k S_j, into k and into S_j */
                    for (i = 0; i < dk; ++i) {
                        double acc = 0.0;
                        for (c = 0; c < dv; ++c) acc += Sa[(size_t)i * dv + c] * (-bj * du[c]);
                        dkj[i] += acc;
                    }
                    for (i = 0; i < dk; ++i)
                        for (c = 0; c < dv; ++c) Hg[(size_t)i * dv + c] -= kj[i] * bj * du[c];
                }
                if (gate == ORACLE_GATE_SCALAR) {
                    double acc = 0.0, a = exp(g[tok]);
                    for (i = 0; i < dk * dv; ++i) acc += Hg[i] * Sj[i];
                    dg[tok] = acc;
                    for (i = 0; i < dk * dv; ++i) Hg[i] = a * Hg[i];
                }
            }
        }
#undef GDP_TOKEN_FWD
        if (ds0) memcpy(ds0 + (size_t)bh * ss, Hg, ss * sizeof(double));
        free(ck); free(Sp); free(Sj); free(Hg); free(St); free(w); free(vh); free(du);
    }
    return failed ? 6 : 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
