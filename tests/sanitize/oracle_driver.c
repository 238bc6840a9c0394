/* Drives the oracle's recurrences on small odd-sized inputs, for sanitizer builds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_mamba2_round_f64(int64_t, int, int, int, double*, const float*, const float*, const float*,
                             const float*, const int32_t*, double*);
void oracle_mamba2_round_f32(int64_t, int, int, int, float*, const float*, const float*, const float*,
                             const float*, const int32_t*, float*);
void oracle_gdn_round_f64(int64_t, int, int, int, double*, const float*, const float*, const float*,
                          const float*, const float*, const int32_t*, double*, double*);
void oracle_gdn_round_f32(int64_t, int, int, int, float*, const float*, const float*, const float*,
                          const float*, const float*, const int32_t*, float*, float*);
void oracle_kda_round_f64(int64_t, int, int, int, double*, const float*, const float*, const float*,
                          const float*, const float*, const int32_t*, double*, double*);
void oracle_kda_round_f32(int64_t, int, int, int, float*, const float*, const float*, const float*,
                          const float*, const float*, const int32_t*, float*, float*);

static float* rnd(size_t n, float lo, float hi) {
  float* p = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * (float)rand() / (float)RAND_MAX;
  return p;
}

int main(void) {
  const int64_t nh = 3;
  const int P = 5, N = 7, T = 3;
  double sum = 0.0;
  for (int round = 0; round < 4; ++round) {
    float* alpha = rnd(nh * T, 0.f, 1.f);
    float* gate = rnd(nh * T * N, 0.f, 1.f);
    float* beta = rnd(nh * T, 0.f, 1.f);
    float* k = rnd(nh * T * N, -1.f, 1.f);
    float* v = rnd(nh * T * P, -1.f, 1.f);
    float* q = rnd(nh * T * N, -1.f, 1.f);
    int32_t acc[3] = {round % (T + 1), T, 0};
    double* S = calloc(nh * P * N, sizeof(double));
    float* Sf = calloc(nh * P * N, sizeof(float));
    double* out = malloc(nh * T * P * sizeof(double));
    double* u = malloc(nh * T * P * sizeof(double));
    float* outf = malloc(nh * T * P * sizeof(float));
    float* uf = malloc(nh * T * P * sizeof(float));
    oracle_mamba2_round_f64(nh, P, N, T, S, alpha, k, v, q, acc, out);
    oracle_mamba2_round_f32(nh, P, N, T, Sf, alpha, k, v, q, acc, outf);
    oracle_gdn_round_f64(nh, P, N, T, S, alpha, beta, k, v, q, acc, out, u);
    oracle_gdn_round_f32(nh, P, N, T, Sf, alpha, beta, k, v, q, acc, outf, uf);
    oracle_kda_round_f64(nh, P, N, T, S, gate, beta, k, v, q, acc, out, u);
    oracle_kda_round_f32(nh, P, N, T, Sf, gate, beta, k, v, q, acc, outf, uf);
    for (int64_t i = 0; i < nh * T * P; ++i) sum += out[i] + u[i] + outf[i] + uf[i];
    free(alpha); free(gate); free(beta); free(k); free(v); free(q);
    free(S); free(Sf); free(out); free(u); free(outf); free(uf);
  }
  printf("checksum %.6f\n", sum);
  return 0;
}
