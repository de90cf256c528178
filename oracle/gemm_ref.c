/*
 * Oracle GEMM: C[i][j] = sum_{k<K} A[i][k] * B[k][j] in IEEE fp64, and in the
 * same pass Abs[i][j] = sum_k |A[i][k]| * |B[k][j]|.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Inputs are the already
 * decoded (dequantised) operand values as fp64, row-major A[M][K], B[K][N].
 * The sum for each (i, j) runs over k = 0, 1, ..., K-1 in that order; the
 * loop over j is innermost only so the rows of B stream contiguously, which
 * changes no element's summation order.  No blocking, no fused multiply-add
 * (built with -ffp-contract=off), no reassociation.
 *
 * Definition: the plain matrix product C = A.B that the persistent kernels of
 * "Work Stealing Scheduler Kernel" (tritonBLAS PR #65) and "[Feature]
 * Introduce tile scheduler" (TileLang PR #2441) compute tile by tile.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void oracle_gemm_f64(const double* A, const double* B, int64_t M, int64_t N,
                     int64_t K, double* C, double* Abs) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    double* c = C + i * N;
    double* s = Abs + i * N;
    for (int64_t j = 0; j < N; ++j) {
      c[j] = 0.0;
      s[j] = 0.0;
    }
    for (int64_t k = 0; k < K; ++k) {
      const double a = A[i * K + k];
      const double aa = fabs(a);
      const double* b = B + k * N;
      for (int64_t j = 0; j < N; ++j) {
        c[j] += a * b[j];
        s[j] += aa * fabs(b[j]);
      }
    }
  }
}

/* Threads the parallel loop above uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
