/*
 * Kimi Delta Attention (KDA) oracle: a plain, slow, obviously correct CPU
 * implementation in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (one head at a time, heads and sequences independent).
 * Sources: "Inside Kimi K3: Architecture of an Open Frontier Model"
 * (academa.ai lecture), sequence paragraph: one state of fixed shape is
 * passed from token to token; its update has two parts, a per-channel
 * diagonal decay (the forget gate) applied to the previous state, then a
 * beta-weighted write that corrects the stored association; the log-decay
 * has a floor of -5.  "Kimi K3" (meridianbulletin.com), section "Handling One
 * Million Tokens with a Fixed-Size State Matrix": S follows the delta rule,
 * beta sets the write strength, alpha the forgetting, and alpha is limited to
 * the interval [e^-5, 1].  "Kimi K3's architecture" (orkas.ai), section "A
 * lower bound that deleted a GPU code path": a single step can shrink the
 * state to no less than e^-5, about 0.67%.
 *
 * The update formula itself is not printed on the pages (it was lost in the
 * text extraction).  The reading used here, token by token, with S a
 * d_k x d_v matrix whose rows are indexed by key channels:
 *
 *     a    = exp(clamp(log_alpha_t, -5, 0))        per key channel
 *     S'   = Diag(a) S                             forget first
 *     e    = v_t - S'^T k_t                        error of the value under k_t
 *     S    = S' + beta_t k_t e^T                   delta write
 *     o_t  = S^T q_t                               read after the write
 *
 * i.e. S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.
 * The decode step is exactly one iteration (T = 1) with S in and out.
 *
 * Layouts (contiguous, row-major), all float64:
 *   q, k, log_alpha : [B, T, H, dk]
 *   v, o            : [B, T, H, dv]
 *   beta            : [B, T, H]
 *   S0, S_T         : [B, H, dk, dv]   (S0 may be NULL: zero initial state)
 *
 * Parallelism: OpenMP over (b, h, block of state columns).  State columns are
 * independent of one another in the recurrence above (column j of S only ever
 * mixes with v_t[j] and o_t[j]), so each unit runs the whole token loop on its
 * own columns.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_LOG_ALPHA_MIN (-5.0)
#define KDA_ORACLE_LOG_ALPHA_MAX (0.0)

/* The bound on the log-decay: log alpha in [-5, 0]. */
static double clamp_log_alpha(double x)
{
    if (x < KDA_ORACLE_LOG_ALPHA_MIN) return KDA_ORACLE_LOG_ALPHA_MIN;
    if (x > KDA_ORACLE_LOG_ALPHA_MAX) return KDA_ORACLE_LOG_ALPHA_MAX;
    return x;
}

int kda_oracle_version(void) { return 1; }

/* Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int kda_oracle_prefill(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const double *S0, double *o, double *S_T,
                       long B, long T, long H, long dk, long dv,
                       long col_block, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return 1;
    if (!o && T > 0) return 1;
    if (col_block <= 0) col_block = 32;
    const long nblk = (dv + col_block - 1) / col_block;
    const long units = B * H * nblk;
    int failed = 0;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long u = 0; u < units; ++u) {
        const long b = u / (H * nblk);
        const long h = (u / nblk) % H;
        const long jb = u % nblk;
        const long j0 = jb * col_block;
        const long j1 = (j0 + col_block < dv) ? j0 + col_block : dv;
        const long w = j1 - j0;

        double *S = (double *)malloc(sizeof(double) * dk * w); /* S[i][j-j0] */
        double *a = (double *)malloc(sizeof(double) * dk);
        double *e = (double *)malloc(sizeof(double) * w);
        if (!S || !a || !e) {
            free(S); free(a); free(e);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }

        /* initial state */
        const double *s0 = S0 ? S0 + (b * H + h) * dk * dv : NULL;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                S[i * w + j] = s0 ? s0[i * dv + j0 + j] : 0.0;

        for (long t = 0; t < T; ++t) {
            const long tok = (b * T + t) * H + h;
            const double *qt = q + tok * dk;
            const double *kt = k + tok * dk;
            const double *lat = log_alpha + tok * dk;
            const double *vt = v + tok * dv;
            const double bt = beta[tok];

            /* forget gate: S' = Diag(a) S */
            for (long i = 0; i < dk; ++i) a[i] = exp(clamp_log_alpha(lat[i]));
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < w; ++j) S[i * w + j] *= a[i];

            /* error of the value stored under k_t: e = v_t - S'^T k_t */
            for (long j = 0; j < w; ++j) e[j] = vt[j0 + j];
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < w; ++j) e[j] -= S[i * w + j] * kt[i];

            /* delta write: S = S' + beta_t k_t e^T */
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < w; ++j) S[i * w + j] += bt * kt[i] * e[j];

            /* read: o_t = S^T q_t */
            double *ot = o + tok * dv;
            for (long j = 0; j < w; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i) acc += S[i * w + j] * qt[i];
                ot[j0 + j] = acc;
            }
        }

        if (S_T) {
            double *st = S_T + (b * H + h) * dk * dv;
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < w; ++j) st[i * dv + j0 + j] = S[i * w + j];
        }
        free(S); free(a); free(e);
    }
    return failed ? 2 : 0;
}
