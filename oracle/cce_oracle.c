/*
 * fp64 CPU oracle for the fused classifier-head + cross-entropy (Cut
 * Cross-Entropy, "CCE").
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the HIP path, and the HIP path never
 * calls it.
 *
 * What it computes is the plain definition of the loss the method reaches
 * exactly (the method's claim is that it never materialises the logits, not
 * that it changes them):
 *
 *   z_iv   = <h_i, e_v>                                   (full logit row)
 *   lse_i  = log sum_v exp(z_iv)
 *   loss_i = lse_i - z_{i,y_i}
 *   g_iv   = dloss_i * (exp(z_iv - lse_i) - [v == y_i])    (d loss / d z_iv)
 *   dH_i   = sum_v g_iv e_v        dE_v = sum_i g_iv h_i
 *
 * Sources: the lit note "The loss and the mask: Cut Cross-Entropy +
 * FlexAttention", section "Contribution" (cross-entropy needs only the
 * correct-token logit, an indexed matmul, and the log-sum-exp over the
 * vocabulary); the CCE paper summary "Cut Your Losses in Large-Vocabulary
 * Language Models", section "Approach" (the backward works from logits
 * recomputed from h and e).  The gradient g is the textbook derivative of
 * log-sum-exp minus an indexed entry.
 *
 * Rows whose label equals ignore_index get loss = lse = 0 and contribute
 * nothing to dH or dE (the pages drop such rows before the head; see the lit
 * note's "What transfers to us").  dloss carries the caller's reduction.
 *
 * Everything is double precision, loops run in ascending index order, and
 * nothing is blocked, fused or reordered beyond the definition above.  The
 * only parallelism is over independent output rows (OpenMP).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

void cce_oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int cce_oracle_max_threads(void) { return omp_get_max_threads(); }

static double dot(const double *a, const double *b, int64_t n)
{
    double s = 0.0;
    for (int64_t k = 0; k < n; ++k) s += a[k] * b[k];
    return s;
}

/*
 * Forward for the listed rows, and (if dH != NULL) their rows of dH.
 * For every listed row i the full logit row z_i. (V doubles) is built,
 * then lse_i, loss_i and dH_i as defined above.
 * rows[r] indexes H / labels / dloss; outputs are indexed by r.
 * Returns 0, or -1 if a buffer cannot be allocated.
 */
int cce_oracle_rows(const double *H, const double *E, const int64_t *labels,
                    const double *dloss, const int64_t *rows, int64_t nrows,
                    int64_t D, int64_t V, int64_t ignore_index,
                    double *lse, double *loss, double *dH)
{
    int fail = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc((size_t)V * sizeof(double));
        if (!z) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!z) continue;
            const int64_t i = rows[r];
            const int64_t y = labels[i];
            if (y == ignore_index) {
                lse[r] = 0.0;
                loss[r] = 0.0;
                if (dH) memset(dH + r * D, 0, (size_t)D * sizeof(double));
                continue;
            }
            const double *h = H + i * D;
            double m = -INFINITY;
            for (int64_t v = 0; v < V; ++v) {
                z[v] = dot(h, E + v * D, D);
                if (z[v] > m) m = z[v];
            }
            double s = 0.0;
            for (int64_t v = 0; v < V; ++v) s += exp(z[v] - m);
            const double l = m + log(s);
            lse[r] = l;
            loss[r] = l - z[y];
            if (dH) {
                double *out = dH + r * D;
                memset(out, 0, (size_t)D * sizeof(double));
                for (int64_t v = 0; v < V; ++v) {
                    const double g = dloss[i] * (exp(z[v] - l) - (v == y ? 1.0 : 0.0));
                    const double *e = E + v * D;
                    for (int64_t d = 0; d < D; ++d) out[d] += g * e[d];
                }
            }
        }
        free(z);
    }
    return fail ? -1 : 0;
}

/*
 * dE_v = sum_i g_iv h_i for the listed vocabulary rows vids[k] (output row k),
 * given lse_i for every row i (as computed by cce_oracle_rows over all rows).
 * Rows are visited in ascending order; each output row is owned by one thread.
 */
int cce_oracle_dE(const double *H, const double *E, const int64_t *labels,
                  const double *lse, const double *dloss, int64_t N,
                  const int64_t *vids, int64_t nv, int64_t D,
                  int64_t ignore_index, double *dE)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t k = 0; k < nv; ++k) {
        const int64_t v = vids[k];
        const double *e = E + v * D;
        double *out = dE + k * D;
        memset(out, 0, (size_t)D * sizeof(double));
        for (int64_t i = 0; i < N; ++i) {
            const int64_t y = labels[i];
            if (y == ignore_index) continue;
            const double *h = H + i * D;
            const double z = dot(h, e, D);
            const double g = dloss[i] * (exp(z - lse[i]) - (v == y ? 1.0 : 0.0));
            for (int64_t d = 0; d < D; ++d) out[d] += g * h[d];
        }
    }
    return 0;
}

/*
 * Mean logit of every vocabulary entry over the non-ignored rows:
 * key_v = (1 / N_valid) sum_{i valid} z_iv, straight from its definition.
 * This is the sort key of the optional vocabulary reordering (the lit note's
 * "Contribution": a vocabulary sort groups the surviving blocks).
 * With no valid row every key is 0.
 */
int cce_oracle_mean_logit(const double *H, const double *E, const int64_t *labels,
                          int64_t N, int64_t D, int64_t V, int64_t ignore_index,
                          double *key)
{
    int64_t nvalid = 0;
    for (int64_t i = 0; i < N; ++i) nvalid += (labels[i] != ignore_index);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t v = 0; v < V; ++v) {
        double s = 0.0;
        for (int64_t i = 0; i < N; ++i)
            if (labels[i] != ignore_index) s += dot(H + i * D, E + v * D, D);
        key[v] = nvalid ? s / (double)nvalid : 0.0;
    }
    return 0;
}
