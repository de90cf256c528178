/* Driver for a sanitizer build of the oracle's C GEMM (oracle/gemm_ref.c,
 * included as is): small shapes, edge sizes among them (empty ones too), each checked element
 * by element against a plain triple loop over the same definition (fp64 sum
 * over k in ascending order, and the |A|.|B| bound), so that AddressSanitizer
 * and UndefinedBehaviorSanitizer see every index the oracle computes.
 * Exits 0 when every case matches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/gemm_ref.c"

static double draw(uint64_t* s) {
  *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
  return (double)(int64_t)(*s >> 40) / (double)(1LL << 23) - 1.0;
}

int main(void) {
  const int64_t sizes[] = {0, 1, 2, 3, 17, 64, 65};  /* 0: empty A, B or C; K = 0 gives C = 0 */
  const int ns = (int)(sizeof(sizes) / sizeof(sizes[0]));
  uint64_t seed = 7;
  int bad = 0;
  for (int a = 0; a < ns; ++a)
    for (int b = 0; b < ns; ++b)
      for (int c = 0; c < ns; ++c) {
        const int64_t M = sizes[a], N = sizes[b], K = sizes[(a + b + c) % ns];
        double* A = malloc(sizeof(double) * M * K);
        double* B = malloc(sizeof(double) * K * N);
        double* C = malloc(sizeof(double) * M * N);
        double* S = malloc(sizeof(double) * M * N);
        for (int64_t i = 0; i < M * K; ++i) A[i] = draw(&seed);
        for (int64_t i = 0; i < K * N; ++i) B[i] = draw(&seed);
        oracle_gemm_f64(A, B, M, N, K, C, S);
        for (int64_t i = 0; i < M; ++i)
          for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
              acc += A[i * K + k] * B[k * N + j];
              abs_acc += fabs(A[i * K + k]) * fabs(B[k * N + j]);
            }
            if (C[i * N + j] != acc || S[i * N + j] != abs_acc) ++bad;
          }
        free(A);
        free(B);
        free(C);
        free(S);
      }
  printf("mismatches: %d\n", bad);
  return bad != 0;
}
