/*
 * Loop-nest fp64 reference of the three products of a linear layer.
 *
 * TEST INFRASTRUCTURE ONLY: built into oracle/libzb_oracle.so and loaded by
 * oracle/loopnest.py for the tests and the benchmark's CPU-baseline leg.
 * Nothing in the product library links or calls it.
 *
 * "Zero-Bubble Pipeline Parallelism Guide for LLMs", section "Core
 * Innovation 1: Mathematical Decomposition of the Backward Pass": a linear
 * layer's forward gives Y from X and W; its backward splits into the input
 * gradient B (needs only dY and W) and the weight gradient W (needs dY and
 * the stashed X), accumulated over microbatches.  With the weight stored
 * [out][in] (row-major, as the library stores it):
 *
 *   F: Y[t][o]   = sum_i X[t][i]  * W[o][i]
 *   B: dX[t][i]  = sum_o dY[t][o] * W[o][i]
 *   W: dW[o][i] += sum_t dY[t][o] * X[t][i]
 *
 * Plain loop nests in double precision, every sum taken in index order,
 * parallel (OpenMP) over the rows of the output only, so each output
 * element is computed by one thread in a fixed order.  No blocking, no
 * reordering of a sum.
 */
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void zbo_linear_fwd(int T, int in, int out, const double* X, const double* W, double* Y) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double* x = X + (size_t)t * in;
        for (int o = 0; o < out; ++o) {
            const double* w = W + (size_t)o * in;
            double s = 0.0;
            for (int i = 0; i < in; ++i) s += x[i] * w[i];
            Y[(size_t)t * out + o] = s;
        }
    }
}

void zbo_linear_bwd_input(int T, int in, int out, const double* dY, const double* W, double* dX) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double* dx = dX + (size_t)t * in;
        for (int i = 0; i < in; ++i) dx[i] = 0.0;
        for (int o = 0; o < out; ++o) {
            const double g = dY[(size_t)t * out + o];
            const double* w = W + (size_t)o * in;
            for (int i = 0; i < in; ++i) dx[i] += g * w[i];
        }
    }
}

void zbo_linear_bwd_weight(int T, int in, int out, const double* dY, const double* X, double* dW) {
#pragma omp parallel for schedule(static)
    for (int o = 0; o < out; ++o) {
        double* dw = dW + (size_t)o * in;
        for (int t = 0; t < T; ++t) {
            const double g = dY[(size_t)t * out + o];
            const double* x = X + (size_t)t * in;
            for (int i = 0; i < in; ++i) dw[i] += g * x[i];
        }
    }
}

int zbo_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
