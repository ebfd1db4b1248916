/*
 * gdr_oracle.c -- plain, slow, obviously correct fp64 CPU model of the gated
 * delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: it is used by the test-suite, by the package's smoke check and by
 * the CPU-baseline leg of the benchmark.  It shares no code, header, helper or
 * constant with the HIP library.
 *
 * What it computes (one token at a time, no chunking, no reassociation):
 *
 *   Gated DeltaNet (per-head scalar decay) -- page "How the New Flash Models
 *   Work: Inside GLM-5.3-Flash and Qwen3.8-Flash-Next", section "Linear
 *   attention: a fixed-size memory in place of the cache", the Gated DeltaNet
 *   equation:   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *               o_t = S_t q_t.
 *   Kimi Delta Attention (per-key-channel decay) -- same page and section, the
 *   KDA equation:  S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T)
 *                        + beta_t v_t k_t^T.
 *
 *   The same section gives each head one state of d_v rows by d_k columns;
 *   the decay multiplies key columns.  Expanding either equation row by
 *   row gives the order used below:
 *       S'   = S_{t-1} Diag(alpha_t)                 (decay)
 *       x    = S' k_t                                (what S' recalls for k_t)
 *       u    = beta_t (v_t - x)                      (erase-then-write)
 *       S_t  = S' + u k_t^T
 *       o_t  = scale * S_t q_t                       (readout after the write)
 *   With alpha_t = 1 this is the ungated delta rule printed on page "Qwen3.8
 *   Flash vs GLM 5.3 Flash: Twin Releases Cement the 3:1 Hybrid Architecture
 *   Era", section "The 3:1 Blueprint: Recurrent Delta Rules and 2048-Token
 *   Indexing".  The pages print no query scale; `scale` is an extra factor on
 *   the readout (1 reproduces the equations exactly).
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q, k        [tokens][H][dk]
 *   v, out      [tokens][H][dv]
 *   beta        [tokens][H]
 *   log_alpha   [tokens][H]        (per_channel_gate == 0, GDN)
 *               [tokens][H][dk]    (per_channel_gate == 1, KDA)
 *   states      [num_seqs][H][dv][dk]
 * Sequence n owns tokens seq_bounds[n] .. seq_bounds[n+1]-1 and starts from
 * initial_state[n] (zeros when initial_state is NULL); the state never crosses
 * a sequence boundary.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (sequence, head) unit, token by token. */
static void run_unit(int64_t n, int64_t h, const int64_t *seq_bounds,
                     int64_t H, int64_t dk, int64_t dv, int per_channel_gate,
                     const double *q, const double *k, const double *v,
                     const double *beta, const double *log_alpha,
                     const double *initial_state, double scale, double *out,
                     double *final_state, double *S, double *alpha) {
    const int64_t state_elems = dv * dk;
    const int64_t unit = n * H + h;
    if (initial_state)
        memcpy(S, initial_state + unit * state_elems, sizeof(double) * state_elems);
    else
        memset(S, 0, sizeof(double) * state_elems);

    for (int64_t t = seq_bounds[n]; t < seq_bounds[n + 1]; ++t) {
        const double *kt = k + (t * H + h) * dk;
        const double *qt = q + (t * H + h) * dk;
        const double *vt = v + (t * H + h) * dv;
        const double bt = beta[t * H + h];
        double *ot = out + (t * H + h) * dv;

        /* alpha_t = exp(log alpha_t): one value per head, or one per key channel */
        for (int64_t j = 0; j < dk; ++j)
            alpha[j] = per_channel_gate ? exp(log_alpha[(t * H + h) * dk + j])
                                        : exp(log_alpha[t * H + h]);

        for (int64_t i = 0; i < dv; ++i) {
            double *row = S + i * dk;
            double x = 0.0;
            for (int64_t j = 0; j < dk; ++j) {
                row[j] *= alpha[j];        /* S' = S Diag(alpha) */
                x += row[j] * kt[j];       /* x_i = (S' k)_i     */
            }
            const double u = bt * (vt[i] - x);
            double o = 0.0;
            for (int64_t j = 0; j < dk; ++j) {
                row[j] += u * kt[j];       /* S = S' + u k^T     */
                o += row[j] * qt[j];       /* (S q)_i            */
            }
            ot[i] = scale * o;
        }
    }
    if (final_state)
        memcpy(final_state + unit * state_elems, S, sizeof(double) * state_elems);
}

/*
 * Returns 0 on success, -1 on an invalid argument, -2 when out of memory.
 * num_threads <= 0 lets OpenMP choose.  Units (sequence, head) run in parallel;
 * each unit is strictly sequential over its tokens.
 */
int gdr_oracle_recurrence(int64_t num_seqs, const int64_t *seq_bounds,
                          int64_t num_heads, int64_t dk, int64_t dv,
                          int per_channel_gate, const double *q, const double *k,
                          const double *v, const double *beta,
                          const double *log_alpha, const double *initial_state,
                          double scale, double *out, double *final_state,
                          int num_threads) {
    if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0 || !seq_bounds)
        return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (seq_bounds[n + 1] < seq_bounds[n]) return -1;
    if (seq_bounds[num_seqs] > seq_bounds[0] && (!q || !k || !v || !beta || !log_alpha || !out))
        return -1;

    const int64_t units = num_seqs * num_heads;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel num_threads(num_threads)
#endif
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(dv * dk));
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!S || !alpha) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < units; ++u) {
            if (!S || !alpha) continue;
            run_unit(u / num_heads, u % num_heads, seq_bounds, num_heads, dk, dv,
                     per_channel_gate, q, k, v, beta, log_alpha, initial_state,
                     scale, out, final_state, S, alpha);
        }
        free(S);
        free(alpha);
    }
    return failed ? -2 : 0;
}

/* Threads OpenMP would use by default (the CPU-baseline reports it). */
int gdr_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Gradients of the recurrence above (reverse mode, one token at a time).
 *
 * The pages describe training these layers but print no backward pass, so
 * this is the plain chain rule applied to the five forward steps, in reverse
 * order.  With G the gradient of the loss with respect to S_t (accumulated
 * from later tokens, or d_final_state after the last token) and dO_t the
 * gradient with respect to o_t:
 *
 *     G     += scale * dO_t q_t^T             (o_t = scale S_t q_t)
 *     dq_t   = scale * S_t^T dO_t
 *     du     = G k_t                          (S_t = S' + u k_t^T)
 *     dk_t   = G^T u
 *     dbeta  = du . (v_t - x)                 (u = beta (v_t - x))
 *     dv_t   = beta du
 *     dx     = -beta du
 *     dS'    = G + dx k_t^T                   (x = S' k_t)
 *     dk_t  += S'^T dx
 *     dlog alpha_t[j] = sum_i dS'[i][j] S'[i][j]   (S' = S_{t-1} Diag(alpha),
 *                                                   d alpha / d log alpha = alpha;
 *                                                   summed over j for one
 *                                                   decay per head)
 *     G_{t-1} = dS' Diag(alpha_t)
 *
 * and d_initial_state = G_0 after the first token.  The forward states each
 * step needs are recomputed: the unit's states are kept every kSegment tokens
 * on a first forward walk, and each segment is re-walked forward (keeping
 * every S_{t-1}) before it is walked backward.
 *
 * d_out has out's layout; d_final_state and d_initial_state the states'
 * layout (d_final_state NULL = zeros; d_initial_state NULL = not written).
 * dq, dk have q's layout; dv v's; dbeta beta's; dlog_alpha log_alpha's.
 * Returns 0, -1 on an invalid argument, -2 when out of memory.
 */
enum { kSegment = 64 };

static void forward_token(const double *S_prev, double *S, int64_t dk, int64_t dv,
                          const double *kt, const double *vt, double bt,
                          const double *alpha) {
    for (int64_t i = 0; i < dv; ++i) {
        const double *prow = S_prev + i * dk;
        double *row = S + i * dk;
        double x = 0.0;
        for (int64_t j = 0; j < dk; ++j) {
            row[j] = prow[j] * alpha[j];
            x += row[j] * kt[j];
        }
        const double u = bt * (vt[i] - x);
        for (int64_t j = 0; j < dk; ++j) row[j] += u * kt[j];
    }
}

static void gate_values(double *alpha, const double *log_alpha, int per_channel_gate,
                        int64_t t, int64_t H, int64_t h, int64_t dk) {
    for (int64_t j = 0; j < dk; ++j)
        alpha[j] = per_channel_gate ? exp(log_alpha[(t * H + h) * dk + j])
                                    : exp(log_alpha[t * H + h]);
}

static int backward_unit(int64_t n, int64_t h, const int64_t *seq_bounds,
                         int64_t H, int64_t dk, int64_t dv, int per_channel_gate,
                         const double *q, const double *k, const double *v,
                         const double *beta, const double *log_alpha,
                         const double *initial_state, double scale,
                         const double *d_out, const double *d_final_state,
                         double *dq, double *dkk, double *dvv, double *dbeta,
                         double *dlog_alpha, double *d_initial_state) {
    const int64_t se = dv * dk;
    const int64_t unit = n * H + h;
    const int64_t t0 = seq_bounds[n], t1 = seq_bounds[n + 1];
    const int64_t len = t1 - t0;
    const int64_t nseg = (len + kSegment - 1) / kSegment;
    /* checkpoints: state before the first token of every segment */
    double *ckpt = (double *)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * se));
    /* states inside one segment: hist[r] = state before token r of the segment,
       hist[kSegment] = after its last token */
    double *hist = (double *)malloc(sizeof(double) * (size_t)((kSegment + 1) * se));
    double *G = (double *)malloc(sizeof(double) * (size_t)se);
    double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
    double *Sp = (double *)malloc(sizeof(double) * (size_t)se);   /* S' of one token */
    double *acc_q = (double *)malloc(sizeof(double) * (size_t)dk);
    double *acc_k = (double *)malloc(sizeof(double) * (size_t)dk);
    double *acc_a = (double *)malloc(sizeof(double) * (size_t)dk);
    int rc = 0;
    if (!ckpt || !hist || !G || !alpha || !Sp || !acc_q || !acc_k || !acc_a) {
        rc = -2;
        goto done;
    }

    /* first forward walk: checkpoints only */
    if (initial_state)
        memcpy(hist, initial_state + unit * se, sizeof(double) * se);
    else
        memset(hist, 0, sizeof(double) * se);
    for (int64_t s = 0; s < nseg; ++s) {
        memcpy(ckpt + s * se, hist, sizeof(double) * se);
        const int64_t a = t0 + s * kSegment, b = a + kSegment < t1 ? a + kSegment : t1;
        for (int64_t t = a; t < b; ++t) {
            gate_values(alpha, log_alpha, per_channel_gate, t, H, h, dk);
            forward_token(hist, hist + se, dk, dv, k + (t * H + h) * dk, v + (t * H + h) * dv,
                          beta[t * H + h], alpha);
            memcpy(hist, hist + se, sizeof(double) * se);
        }
    }

    if (d_final_state)
        memcpy(G, d_final_state + unit * se, sizeof(double) * se);
    else
        memset(G, 0, sizeof(double) * se);

    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t a = t0 + s * kSegment, b = a + kSegment < t1 ? a + kSegment : t1;
        memcpy(hist, ckpt + s * se, sizeof(double) * se);
        for (int64_t t = a; t < b; ++t) {
            gate_values(alpha, log_alpha, per_channel_gate, t, H, h, dk);
            forward_token(hist + (t - a) * se, hist + (t - a + 1) * se, dk, dv,
                          k + (t * H + h) * dk, v + (t * H + h) * dv, beta[t * H + h], alpha);
        }
        for (int64_t t = b - 1; t >= a; --t) {
            const double *S_prev = hist + (t - a) * se;      /* S_{t-1} */
            const double *S_t = hist + (t - a + 1) * se;     /* S_t     */
            const double *kt = k + (t * H + h) * dk;
            const double *qt = q + (t * H + h) * dk;
            const double *vt = v + (t * H + h) * dv;
            const double *dot = d_out + (t * H + h) * dv;
            const double bt = beta[t * H + h];
            gate_values(alpha, log_alpha, per_channel_gate, t, H, h, dk);
            for (int64_t j = 0; j < dk; ++j) acc_q[j] = acc_k[j] = acc_a[j] = 0.0;
            double db = 0.0;
            for (int64_t i = 0; i < dv; ++i) {
                double *g = G + i * dk;
                const double *sp = S_prev + i * dk;
                const double *st = S_t + i * dk;
                double *spr = Sp + i * dk;
                /* S' row and x_i = (S' k)_i, u_i */
                double x = 0.0;
                for (int64_t j = 0; j < dk; ++j) {
                    spr[j] = sp[j] * alpha[j];
                    x += spr[j] * kt[j];
                }
                const double u = bt * (vt[i] - x);
                /* total gradient of S_t row i, and the readout's dq */
                double du = 0.0;
                for (int64_t j = 0; j < dk; ++j) {
                    g[j] += scale * dot[i] * qt[j];
                    acc_q[j] += scale * st[j] * dot[i];
                    du += g[j] * kt[j];
                }
                db += du * (vt[i] - x);
                dvv[(t * H + h) * dv + i] = bt * du;
                const double dx = -bt * du;
                for (int64_t j = 0; j < dk; ++j) {
                    acc_k[j] += g[j] * u + spr[j] * dx;
                    const double dsp = g[j] + dx * kt[j];      /* dS'[i][j] */
                    acc_a[j] += dsp * spr[j];
                    g[j] = dsp * alpha[j];                    /* G_{t-1}   */
                }
            }
            dbeta[t * H + h] = db;
            double a_sum = 0.0;
            for (int64_t j = 0; j < dk; ++j) {
                dq[(t * H + h) * dk + j] = acc_q[j];
                dkk[(t * H + h) * dk + j] = acc_k[j];
                if (per_channel_gate)
                    dlog_alpha[(t * H + h) * dk + j] = acc_a[j];
                a_sum += acc_a[j];
            }
            if (!per_channel_gate) dlog_alpha[t * H + h] = a_sum;
        }
    }
    if (d_initial_state) memcpy(d_initial_state + unit * se, G, sizeof(double) * se);
done:
    free(ckpt); free(hist); free(G); free(alpha); free(Sp);
    free(acc_q); free(acc_k); free(acc_a);
    return rc;
}

int gdr_oracle_recurrence_backward(int64_t num_seqs, const int64_t *seq_bounds,
                                   int64_t num_heads, int64_t dk, int64_t dv,
                                   int per_channel_gate, const double *q, const double *k,
                                   const double *v, const double *beta,
                                   const double *log_alpha, const double *initial_state,
                                   double scale, const double *d_out,
                                   const double *d_final_state, double *dq, double *dkk,
                                   double *dvv, double *dbeta, double *dlog_alpha,
                                   double *d_initial_state, int num_threads) {
    if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0 || !seq_bounds)
        return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (seq_bounds[n + 1] < seq_bounds[n]) return -1;
    if (seq_bounds[num_seqs] > seq_bounds[0] &&
        (!q || !k || !v || !beta || !log_alpha || !d_out || !dq || !dkk || !dvv || !dbeta || !dlog_alpha))
        return -1;
    const int64_t units = num_seqs * num_heads;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int rc = backward_unit(u / num_heads, u % num_heads, seq_bounds, num_heads, dk, dv,
                                     per_channel_gate, q, k, v, beta, log_alpha, initial_state,
                                     scale, d_out, d_final_state, dq, dkk, dvv, dbeta,
                                     dlog_alpha, d_initial_state);
        if (rc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = rc;
        }
    }
    return failed;
}
