/*
 * CPU oracle for the ReplaySSM decode path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library. The product path (the HIP library under ssm_decode_amd/) never
 * calls it, shares no code with it, and this file includes nothing of it.
 *
 * What it computes is the plain, eager, token-by-token SSM recurrence: the
 * definition that ReplaySSM claims to reproduce "up to floating-point
 * differences" ("ReplaySSM: Cache SSM Inputs, Not State", Limits; the paper
 * abstract on the Lattice page says the method unrolls this recurrence into a
 * checkpoint plus buffered inputs). No replay, no checkpoint, no buffer, no
 * blocking: every token updates the full state and reads the output from it.
 *
 *   Mamba-2   S_t = alpha_t * S_{t-1} + v_t k_t^T            o_t = S_t q_t
 *   GDN       S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T)
 *                   + beta_t v_t k_t^T                        o_t = S_t q_t
 *   KDA       S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T)
 *                   + beta_t v_t k_t^T                        o_t = S_t q_t
 *             (Kimi Delta Attention: the gate a_t is a vector over the key
 *             channels; the summary page names it compatible in principle,
 *             Limits, without a formula; this is the delta rule with GDN's
 *             scalar gate replaced by a per-channel one, see the design notes)
 *
 * The GDN form is the gated delta rule in the convention fixed by the
 * correction term u_t = beta_t (v_t - alpha_t S_{t-1} k_t) that the summary
 * page gives ("How it works", Gated DeltaNet): expanding
 * alpha_t S_{t-1} + u_t k_t^T gives exactly the line above, so alpha_t also
 * scales the erased component. The oracle evaluates the delta rule itself, in
 * the order written (first w = S_{t-1} k_t, then the update), and reports u_t
 * from that same w only so that the GPU's stored correction records can be
 * compared.
 *
 * Speculative rounds ("How it works", Speculative decoding; the flowchart):
 * from the committed state the T drafts are applied one after another, every
 * draft's output is recorded, and the committed state advances by the accepted
 * prefix only (acc = T in standard decoding, where T = 1).
 *
 * Layouts (row-major, one entry per head; heads are independent):
 *   S     [nh][P][N]       committed state (in/out)
 *   alpha [nh][T], beta [nh][T]   (KDA: alpha [nh][T][N])
 *   k, q  [nh][T][N],  v [nh][T][P]
 *   acc   [nh]             accepted prefix length in 0..T
 *   out   [nh][T][P]       o for every draft
 *   u     [nh][T][P]       GDN correction of every draft (may be NULL)
 *
 * Precision: the _f64 functions keep the state and all arithmetic in double
 * (the reference for parity); the _f32 functions do the same in float, only to
 * bound the oracle's own rounding.
 *
 * Parallelism: OpenMP over heads only; each head runs the loops above exactly.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- Mamba-2 */

void oracle_mamba2_round_f64(int64_t nh, int P, int N, int T, double* S,
                             const float* alpha, const float* k, const float* v,
                             const float* q, const int32_t* acc, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t hd = 0; hd < nh; ++hd) {
    double* Sc = S + hd * (int64_t)P * N;
    double* W = (double*)malloc(sizeof(double) * (size_t)P * N);
    memcpy(W, Sc, sizeof(double) * (size_t)P * N);
    for (int i = 0; i < T; ++i) {
      const double a = alpha[hd * T + i];
      const float* ki = k + (hd * T + i) * (int64_t)N;
      const float* vi = v + (hd * T + i) * (int64_t)P;
      const float* qi = q + (hd * T + i) * (int64_t)N;
      for (int r = 0; r < P; ++r)
        for (int c = 0; c < N; ++c)
          W[r * N + c] = a * W[r * N + c] + (double)vi[r] * (double)ki[c];
      double* oi = out + (hd * T + i) * (int64_t)P;
      for (int r = 0; r < P; ++r) {
        double s = 0.0;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * (double)qi[c];
        oi[r] = s;
      }
      if (i + 1 == acc[hd]) memcpy(Sc, W, sizeof(double) * (size_t)P * N);
    }
    free(W);
  }
}

void oracle_mamba2_round_f32(int64_t nh, int P, int N, int T, float* S,
                             const float* alpha, const float* k, const float* v,
                             const float* q, const int32_t* acc, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t hd = 0; hd < nh; ++hd) {
    float* Sc = S + hd * (int64_t)P * N;
    float* W = (float*)malloc(sizeof(float) * (size_t)P * N);
    memcpy(W, Sc, sizeof(float) * (size_t)P * N);
    for (int i = 0; i < T; ++i) {
      const float a = alpha[hd * T + i];
      const float* ki = k + (hd * T + i) * (int64_t)N;
      const float* vi = v + (hd * T + i) * (int64_t)P;
      const float* qi = q + (hd * T + i) * (int64_t)N;
      for (int r = 0; r < P; ++r)
        for (int c = 0; c < N; ++c)
          W[r * N + c] = a * W[r * N + c] + vi[r] * ki[c];
      float* oi = out + (hd * T + i) * (int64_t)P;
      for (int r = 0; r < P; ++r) {
        float s = 0.0f;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * qi[c];
        oi[r] = s;
      }
      if (i + 1 == acc[hd]) memcpy(Sc, W, sizeof(float) * (size_t)P * N);
    }
    free(W);
  }
}

/* -------------------------------------------------------- Gated DeltaNet */

void oracle_gdn_round_f64(int64_t nh, int P, int N, int T, double* S,
                          const float* alpha, const float* beta, const float* k,
                          const float* v, const float* q, const int32_t* acc,
                          double* out, double* u) {
#pragma omp parallel for schedule(static)
  for (int64_t hd = 0; hd < nh; ++hd) {
    double* Sc = S + hd * (int64_t)P * N;
    double* W = (double*)malloc(sizeof(double) * (size_t)P * N);
    double* w = (double*)malloc(sizeof(double) * (size_t)P);
    memcpy(W, Sc, sizeof(double) * (size_t)P * N);
    for (int i = 0; i < T; ++i) {
      const double a = alpha[hd * T + i];
      const double b = beta[hd * T + i];
      const float* ki = k + (hd * T + i) * (int64_t)N;
      const float* vi = v + (hd * T + i) * (int64_t)P;
      const float* qi = q + (hd * T + i) * (int64_t)N;
      /* w = S_{t-1} k_t */
      for (int r = 0; r < P; ++r) {
        double s = 0.0;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * (double)ki[c];
        w[r] = s;
      }
      /* S_t = alpha (S_{t-1} - beta w k^T) + beta v k^T */
      for (int r = 0; r < P; ++r)
        for (int c = 0; c < N; ++c)
          W[r * N + c] = a * (W[r * N + c] - b * w[r] * (double)ki[c]) +
                         b * (double)vi[r] * (double)ki[c];
      double* oi = out + (hd * T + i) * (int64_t)P;
      for (int r = 0; r < P; ++r) {
        double s = 0.0;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * (double)qi[c];
        oi[r] = s;
      }
      if (u) {
        double* ui = u + (hd * T + i) * (int64_t)P;
        for (int r = 0; r < P; ++r) ui[r] = b * ((double)vi[r] - a * w[r]);
      }
      if (i + 1 == acc[hd]) memcpy(Sc, W, sizeof(double) * (size_t)P * N);
    }
    free(w);
    free(W);
  }
}

void oracle_gdn_round_f32(int64_t nh, int P, int N, int T, float* S,
                          const float* alpha, const float* beta, const float* k,
                          const float* v, const float* q, const int32_t* acc,
                          float* out, float* u) {
#pragma omp parallel for schedule(static)
  for (int64_t hd = 0; hd < nh; ++hd) {
    float* Sc = S + hd * (int64_t)P * N;
    float* W = (float*)malloc(sizeof(float) * (size_t)P * N);
    float* w = (float*)malloc(sizeof(float) * (size_t)P);
    memcpy(W, Sc, sizeof(float) * (size_t)P * N);
    for (int i = 0; i < T; ++i) {
      const float a = alpha[hd * T + i];
      const float b = beta[hd * T + i];
      const float* ki = k + (hd * T + i) * (int64_t)N;
      const float* vi = v + (hd * T + i) * (int64_t)P;
      const float* qi = q + (hd * T + i) * (int64_t)N;
      for (int r = 0; r < P; ++r) {
        float s = 0.0f;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * ki[c];
        w[r] = s;
      }
      for (int r = 0; r < P; ++r)
        for (int c = 0; c < N; ++c)
          W[r * N + c] = a * (W[r * N + c] - b * w[r] * ki[c]) + b * vi[r] * ki[c];
      float* oi = out + (hd * T + i) * (int64_t)P;
      for (int r = 0; r < P; ++r) {
        float s = 0.0f;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * qi[c];
        oi[r] = s;
      }
      if (u) {
        float* ui = u + (hd * T + i) * (int64_t)P;
        for (int r = 0; r < P; ++r) ui[r] = b * (vi[r] - a * w[r]);
      }
      if (i + 1 == acc[hd]) memcpy(Sc, W, sizeof(float) * (size_t)P * N);
    }
    free(w);
    free(W);
  }
}

/* ------------------------------------------------- Kimi Delta Attention */

void oracle_kda_round_f64(int64_t nh, int P, int N, int T, double* S,
                          const float* alpha, const float* beta, const float* k,
                          const float* v, const float* q, const int32_t* acc,
                          double* out, double* u) {
#pragma omp parallel for schedule(static)
  for (int64_t hd = 0; hd < nh; ++hd) {
    double* Sc = S + hd * (int64_t)P * N;
    double* W = (double*)malloc(sizeof(double) * (size_t)P * N);
    double* w = (double*)malloc(sizeof(double) * (size_t)P);
    memcpy(W, Sc, sizeof(double) * (size_t)P * N);
    for (int i = 0; i < T; ++i) {
      const float* ai = alpha + (hd * T + i) * (int64_t)N;
      const double b = beta[hd * T + i];
      const float* ki = k + (hd * T + i) * (int64_t)N;
      const float* vi = v + (hd * T + i) * (int64_t)P;
      const float* qi = q + (hd * T + i) * (int64_t)N;
      /* w = S_{t-1} Diag(a) k_t */
      for (int r = 0; r < P; ++r) {
        double s = 0.0;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * (double)ai[c] * (double)ki[c];
        w[r] = s;
      }
      /* S_t = S_{t-1} Diag(a) - beta w k^T + beta v k^T */
      for (int r = 0; r < P; ++r)
        for (int c = 0; c < N; ++c)
          W[r * N + c] = W[r * N + c] * (double)ai[c] - b * w[r] * (double)ki[c] +
                         b * (double)vi[r] * (double)ki[c];
      double* oi = out + (hd * T + i) * (int64_t)P;
      for (int r = 0; r < P; ++r) {
        double s = 0.0;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * (double)qi[c];
        oi[r] = s;
      }
      if (u) {
        double* ui = u + (hd * T + i) * (int64_t)P;
        for (int r = 0; r < P; ++r) ui[r] = b * ((double)vi[r] - w[r]);
      }
      if (i + 1 == acc[hd]) memcpy(Sc, W, sizeof(double) * (size_t)P * N);
    }
    free(w);
    free(W);
  }
}

void oracle_kda_round_f32(int64_t nh, int P, int N, int T, float* S,
                          const float* alpha, const float* beta, const float* k,
                          const float* v, const float* q, const int32_t* acc,
                          float* out, float* u) {
#pragma omp parallel for schedule(static)
  for (int64_t hd = 0; hd < nh; ++hd) {
    float* Sc = S + hd * (int64_t)P * N;
    float* W = (float*)malloc(sizeof(float) * (size_t)P * N);
    float* w = (float*)malloc(sizeof(float) * (size_t)P);
    memcpy(W, Sc, sizeof(float) * (size_t)P * N);
    for (int i = 0; i < T; ++i) {
      const float* ai = alpha + (hd * T + i) * (int64_t)N;
      const float b = beta[hd * T + i];
      const float* ki = k + (hd * T + i) * (int64_t)N;
      const float* vi = v + (hd * T + i) * (int64_t)P;
      const float* qi = q + (hd * T + i) * (int64_t)N;
      for (int r = 0; r < P; ++r) {
        float s = 0.0f;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * ai[c] * ki[c];
        w[r] = s;
      }
      for (int r = 0; r < P; ++r)
        for (int c = 0; c < N; ++c)
          W[r * N + c] = W[r * N + c] * ai[c] - b * w[r] * ki[c] + b * vi[r] * ki[c];
      float* oi = out + (hd * T + i) * (int64_t)P;
      for (int r = 0; r < P; ++r) {
        float s = 0.0f;
        for (int c = 0; c < N; ++c) s += W[r * N + c] * qi[c];
        oi[r] = s;
      }
      if (u) {
        float* ui = u + (hd * T + i) * (int64_t)P;
        for (int r = 0; r < P; ++r) ui[r] = b * (vi[r] - w[r]);
      }
      if (i + 1 == acc[hd]) memcpy(Sc, W, sizeof(float) * (size_t)P * N);
    }
    free(w);
    free(W);
  }
}

/* Thread count the OpenMP runtime will use (reported by the CPU baseline). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

/* Sets the thread count of the following oracle calls (the CPU baseline runs at one core too). */
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
