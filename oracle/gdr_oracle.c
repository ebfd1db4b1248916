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
