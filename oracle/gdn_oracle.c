/*
 * fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, header or constant with the
 * HIP path.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
 *        §2.1 delta-rule update, first (unexpanded) form:
 *             S_t = S_{t-1} - beta_t (S_{t-1} k_t - v_t) k_t^T
 *        §2.2 a gate in (0,1) scales the old state (here: a scalar alpha_t per
 *             token that multiplies the whole transition, the write is not
 *             decayed)
 *        §1.3 / §5.3 the naive per-token loop is the correctness baseline.
 *   [P3] "线性注意力机制与Gated DeltaNet的优化实践"
 *        §2.1 the output of token i includes token i itself (inclusive sum),
 *             so o_t is read from the state after the update.
 *
 * What it computes, per (b,h) independently, in fp64, token by token:
 *     S <- alpha_t * S                 (gated decay)
 *     r <- S k_t                       (what the memory returns for k_t)
 *     u <- beta_t * (v_t - r)          (delta-rule error)
 *     S <- S + u k_t^T                 (rank-1 erase + write)
 *     o_t <- S q_t
 * which equals S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 * o_t = S_t q_t, with S stored d_v x d_k (row i = value index, column j = key
 * index).
 *
 * Every input is read as given (fp32; bf16 tensors are passed as their exact
 * fp32 values) and widened to fp64 exactly.  Outputs are fp64.
 *
 * Layouts (all row-major, contiguous):
 *   q, k : [B,H,T,dk]      v : [B,H,T,dv]
 *   alpha, beta : [B,H,T]
 *   s0   : [B,H,dv,dk] or NULL (zero initial state)
 *   o    : [B,H,T,dv]  (out)      sT : [B,H,dv,dk] (out, may be NULL)
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on a single (b,h) state S (dv x dk, fp64). */
static void oracle_token(double* S, int64_t dk, int64_t dv,
                         const float* q, const float* k, const float* v,
                         double alpha, double beta, double* o, double* kd,
                         double* qd) {
    for (int64_t j = 0; j < dk; ++j) {
        kd[j] = (double)k[j];
        qd[j] = (double)q[j];
    }
    for (int64_t i = 0; i < dv; ++i) {
        double* row = S + i * dk;
        /* gated decay of the old state */
        for (int64_t j = 0; j < dk; ++j) row[j] *= alpha;
        /* retrieve with the current key */
        double r = 0.0;
        for (int64_t j = 0; j < dk; ++j) r += row[j] * kd[j];
        /* delta-rule error and rank-1 update of this row */
        double u = beta * ((double)v[i] - r);
        for (int64_t j = 0; j < dk; ++j) row[j] += u * kd[j];
        /* output reads the updated state */
        double acc = 0.0;
        for (int64_t j = 0; j < dk; ++j) acc += row[j] * qd[j];
        o[i] = acc;
    }
}

int gdn_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Full forward pass over T tokens.  Returns 0 on success, 1 on bad args,
 * 2 on allocation failure. */
int gdn_oracle_fwd(const float* q, const float* k, const float* v,
                   const float* alpha, const float* beta, const float* s0,
                   double* o, double* sT, int64_t B, int64_t H, int64_t T,
                   int64_t dk, int64_t dv) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
    if (!o && T > 0) return 1;
    const int64_t chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < chains; ++c) {
        double* S = (double*)malloc(sizeof(double) * (size_t)(dv * dk));
        double* kd = (double*)malloc(sizeof(double) * (size_t)dk);
        double* qd = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!S || !kd || !qd) {
            free(S); free(kd); free(qd);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        if (s0) {
            const float* s = s0 + c * dv * dk;
            for (int64_t e = 0; e < dv * dk; ++e) S[e] = (double)s[e];
        } else {
            memset(S, 0, sizeof(double) * (size_t)(dv * dk));
        }
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = c * T + t;
            oracle_token(S, dk, dv, q + tok * dk, k + tok * dk, v + tok * dv,
                         (double)alpha[tok], (double)beta[tok], o + tok * dv,
                         kd, qd);
        }
        if (sT) memcpy(sT + c * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        free(S); free(kd); free(qd);
    }
    return failed ? 2 : 0;
}

/* One decode step: one token per (n,h), state updated in place (fp64).
 * q,k: [N,H,dk]  v: [N,H,dv]  alpha,beta: [N,H]  state: [N,H,dv,dk]
 * o: [N,H,dv] (out). */
int gdn_oracle_step(const float* q, const float* k, const float* v,
                    const float* alpha, const float* beta, double* state,
                    double* o, int64_t N, int64_t H, int64_t dk, int64_t dv) {
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0 || !state || !o) return 1;
    const int64_t chains = N * H;
    int failed = 0;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < chains; ++c) {
        double* kd = (double*)malloc(sizeof(double) * (size_t)dk);
        double* qd = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!kd || !qd) {
            free(kd); free(qd);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        oracle_token(state + c * dv * dk, dk, dv, q + c * dk, k + c * dk,
                     v + c * dv, (double)alpha[c], (double)beta[c], o + c * dv,
                     kd, qd);
        free(kd); free(qd);
    }
    return failed ? 2 : 0;
}

/*
 * Gated linear attention without the delta rule ([P3] §2.3: the state decays
 * by a gate and gains the outer product of the token's key and value, with no
 * erase term).  In the orientation used above (S is d_v x d_k, row i = value
 * index):  S_t = alpha_t S_{t-1} + beta_t v_t k_t^T,  o_t = S_t q_t,  token by
 * token in fp64:
 *     S <- alpha_t * S
 *     S <- S + beta_t v_t k_t^T
 *     o_t <- S q_t
 * Same layouts and return codes as gdn_oracle_fwd.
 */
int gla_oracle_fwd(const float* q, const float* k, const float* v,
                   const float* alpha, const float* beta, const float* s0,
                   double* o, double* sT, int64_t B, int64_t H, int64_t T,
                   int64_t dk, int64_t dv) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
    if (!o && T > 0) return 1;
    const int64_t chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < chains; ++c) {
        double* S = (double*)malloc(sizeof(double) * (size_t)(dv * dk));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        if (s0) {
            const float* s = s0 + c * dv * dk;
            for (int64_t e = 0; e < dv * dk; ++e) S[e] = (double)s[e];
        } else {
            memset(S, 0, sizeof(double) * (size_t)(dv * dk));
        }
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = c * T + t;
            const float* qt = q + tok * dk;
            const float* kt = k + tok * dk;
            const double a = (double)alpha[tok], b = (double)beta[tok];
            for (int64_t i = 0; i < dv; ++i) {
                double* row = S + i * dk;
                const double w = b * (double)v[tok * dv + i];
                double acc = 0.0;
                for (int64_t j = 0; j < dk; ++j) {
                    row[j] = a * row[j] + w * (double)kt[j];
                    acc += row[j] * (double)qt[j];
                }
                o[tok * dv + i] = acc;
            }
        }
        if (sT) memcpy(sT + c * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        free(S);
    }
    return failed ? 2 : 0;
}

/*
 * The delta rule with a per-dimension gate ([P1] §2.2: the gate may be a
 * vector instead of a scalar).  Reading: alpha_t in (0,1]^{d_k} decays the
 * key columns of the state (S is d_v x d_k), i.e.
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * token by token in fp64:
 *     S[i][j] <- alpha_t[j] * S[i][j]
 *     r <- S k_t;  u <- beta_t (v_t - r);  S <- S + u k_t^T;  o_t <- S q_t
 * alpha is [B,H,T,dk]; everything else as in gdn_oracle_fwd.
 */
int gdn_oracle_fwd_vecgate(const float* q, const float* k, const float* v,
                           const float* alpha, const float* beta, const float* s0,
                           double* o, double* sT, int64_t B, int64_t H, int64_t T,
                           int64_t dk, int64_t dv) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
    if (!o && T > 0) return 1;
    const int64_t chains = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < chains; ++c) {
        double* S = (double*)malloc(sizeof(double) * (size_t)(dv * dk));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        if (s0) {
            const float* s = s0 + c * dv * dk;
            for (int64_t e = 0; e < dv * dk; ++e) S[e] = (double)s[e];
        } else {
            memset(S, 0, sizeof(double) * (size_t)(dv * dk));
        }
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = c * T + t;
            const float* qt = q + tok * dk;
            const float* kt = k + tok * dk;
            const float* at = alpha + tok * dk;
            const double bt = (double)beta[tok];
            for (int64_t i = 0; i < dv; ++i) {
                double* row = S + i * dk;
                double r = 0.0;
                for (int64_t j = 0; j < dk; ++j) {
                    row[j] *= (double)at[j];
                    r += row[j] * (double)kt[j];
                }
                const double u = bt * ((double)v[tok * dv + i] - r);
                double acc = 0.0;
                for (int64_t j = 0; j < dk; ++j) {
                    row[j] += u * (double)kt[j];
                    acc += row[j] * (double)qt[j];
                }
                o[tok * dv + i] = acc;
            }
        }
        if (sT) memcpy(sT + c * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        free(S);
    }
    return failed ? 2 : 0;
}

