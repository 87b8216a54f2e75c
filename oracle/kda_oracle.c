/* Reference (oracle) token loop in plain C -- TEST INFRASTRUCTURE ONLY.
 *
 * The same definition as oracle/kda_oracle.py, written in C so that whole sequences of a
 * million tokens can be checked in seconds: for each selected (sequence, head) unit, every
 * token applies Kimi K3: Open Frontier Intelligence, §2.1.1, eq. (1):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
 *
 * evaluated as: decay the rows of S by exp(g_t) (decay before the delta update), form
 * u = beta_t (v_t - S^T k_t) against the decayed state, add k_t u^T, read out S^T q_t after the
 * update.  All arithmetic is double precision; inputs are upcast from their stored dtype
 * (bf16 bit patterns or float32; g may also be float64, e.g. the decay map of eq. (5) evaluated
 * in double).  Only tests/, the smoke check in __graft_entry__.py and bench.py's CPU-baseline
 * leg load this library; the HIP product path never does, and the two share no code.
 *
 * Units run in parallel with OpenMP (one unit per thread at a time); within a unit the loop is
 * sequential and unblocked.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes: 0 bf16, 1 float32, 2 float64 */
static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == 2) return ((const double*)base)[idx];
    if (dtype == 0) { /* bf16: the 16 stored bits are the top half of a float32 */
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[idx];
}

int kda_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* unit_desc: n_units rows of {b, bos, eos, h, o_offset}.  Token t of row b, head h, channel c
 * lives at ((b * T + t) * H + h) * d + c.  beta at (b * T + t) * H + h.
 * S0_units / ST_out: [n_units, dk, dv] row-major.  o_out: unit u's outputs start at
 * o_offset[u] * dv, one row of dv per token of the unit. */
void kda_oracle_units(const void* q, const void* k, const void* v, const void* g,
                      const void* beta, int in_dtype, int beta_dtype, int g_dtype, int64_t T,
                      int32_t H,
                      int32_t dk, int32_t dv, double scale, int32_t n_units,
                      const int64_t* unit_desc, const double* S0_units, double* o_out,
                      double* ST_out) {
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* at = (double*)malloc(sizeof(double) * (size_t)dk);
        double* y = (double*)malloc(sizeof(double) * (size_t)dv);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
        for (int32_t un = 0; un < n_units; ++un) {
            const int64_t b = unit_desc[5 * un + 0], bos = unit_desc[5 * un + 1];
            const int64_t eos = unit_desc[5 * un + 2], h = unit_desc[5 * un + 3];
            const int64_t ooff = unit_desc[5 * un + 4];
            memcpy(S, S0_units + (size_t)un * dk * dv, sizeof(double) * (size_t)dk * dv);
            for (int64_t t = bos; t < eos; ++t) {
                const int64_t row = (b * T + t) * H + h;
                for (int32_t i = 0; i < dk; ++i) {
                    qt[i] = scale * load_elem(q, in_dtype, row * dk + i);
                    kt[i] = load_elem(k, in_dtype, row * dk + i);
                    at[i] = exp(load_elem(g, g_dtype, row * dk + i));
                }
                const double bt = load_elem(beta, beta_dtype, row);
                /* decay, then y = S^T k on the decayed state */
                for (int32_t j = 0; j < dv; ++j) y[j] = 0.0;
                for (int32_t i = 0; i < dk; ++i) {
                    double* Si = S + (size_t)i * dv;
                    for (int32_t j = 0; j < dv; ++j) {
                        Si[j] *= at[i];
                        y[j] += kt[i] * Si[j];
                    }
                }
                for (int32_t j = 0; j < dv; ++j)
                    u[j] = bt * (load_elem(v, in_dtype, row * dv + j) - y[j]);
                /* rank-one write, then read-out o = S^T q after the update */
                double* ot = o_out + (size_t)(ooff + (t - bos)) * dv;
                for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
                for (int32_t i = 0; i < dk; ++i) {
                    double* Si = S + (size_t)i * dv;
                    for (int32_t j = 0; j < dv; ++j) {
                        Si[j] += kt[i] * u[j];
                        ot[j] += qt[i] * Si[j];
                    }
                }
            }
            memcpy(ST_out + (size_t)un * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        }
        free(S); free(qt); free(kt); free(at); free(y); free(u);
    }
}
