// Eager comparison kernels of libreplayssm: the conventional decode step that
// loads the state, updates it, reads the output from it and stores it back on
// every token ("ReplaySSM: Cache SSM Inputs, Not State", What it claims: a
// conventional step both loads and stores the state). In the speculative form
// every draft's state is stored, one snapshot per draft, which is what a
// conventional engine keeps to be able to roll back (the thread's post [3/N]).
//
// Same private fp32 tile layout and workgroup shape as the replay kernel: one
// workgroup per (sequence, head), one wavefront per 16-row tile, so every
// wavefront holds complete rows and all reductions stay inside it.
#include "device.hpp"

namespace rs {

template <int KIND, int NT>
__global__ void __launch_bounds__(1024) eager_kernel(const EagerArgs a) {
  constexpr int DK = NT * 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int H = a.H, dv = a.dv, T = a.T, ns = a.nslots;
  const int b = blockIdx.x / H;
  const int hd = blockIdx.x - b * H;
  const int64_t bh = (int64_t)b * H + hd;
  const int prow = wave * 16 + col;
  const int64_t hsz = (int64_t)dv * DK;
  float* pool = a.S + bh * ns * hsz + (int64_t)(wave * NT) * 256 + lane * 4;

  int s0 = a.slot ? a.slot[b] : 0;
  if (s0 < 0 || s0 >= ns) s0 = 0;  // never address outside the pool
  f32x4 S[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) S[nt] = ld4_stream(pool + s0 * hsz + nt * 256);

  for (int i = 0; i < T; ++i) {
    const int64_t tok = ((int64_t)b * T + i) * H + hd;
    const float al = KIND == REPLAYSSM_KDA ? 1.f : a.alpha[tok];
    const float* kin = a.k + tok * DK + 4 * g;
    const float* qin = a.q + tok * DK + 4 * g;
    f32x4 kf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) kf[nt] = ld4(kin + nt * 16);
    const float vp = a.v[tok * dv + prow];
    float coef = vp;
    if (KIND == REPLAYSSM_GDN) {
      float w = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w += dot4(S[nt], kf[nt]);
      w = sum_groups(w);
      coef = a.beta[tok] * (vp - al * w);  // u = beta (v - alpha S k)
    }
    if constexpr (KIND == REPLAYSSM_KDA) {
      // per-channel gate: w = S (a * k), u = beta (v - w), S <- S Diag(a) + u k^T
      const float* ain = a.alpha + tok * DK + 4 * g;
      float w = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w += dot4(S[nt], ld4(ain + nt * 16) * kf[nt]);
      w = sum_groups(w);
      coef = a.beta[tok] * (vp - w);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S[nt] *= ld4(ain + nt * 16);
    }
    float o = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      S[nt] = al * S[nt] + coef * kf[nt];
      o += dot4(S[nt], ld4(qin + nt * 16));
    }
    o = sum_groups(o);
    if (g == 0) a.out[tok * dv + prow] = o;
    int sl = s0 + i + 1;
    while (sl >= ns) sl -= ns;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) st4_stream(pool + sl * hsz + nt * 256, S[nt]);
  }
}

template <int KIND>
static hipError_t launch_kind(int dk, const EagerArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.H)), block((unsigned)(a.dv / 16 * kWave));
  switch (dk) {
    case 16: hipLaunchKernelGGL((eager_kernel<KIND, 1>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((eager_kernel<KIND, 2>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((eager_kernel<KIND, 4>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((eager_kernel<KIND, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_eager(int kind, int dk, const EagerArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  if (kind == REPLAYSSM_KDA) return launch_kind<REPLAYSSM_KDA>(dk, a, s);
  return kind == REPLAYSSM_GDN ? launch_kind<REPLAYSSM_GDN>(dk, a, s)
                               : launch_kind<REPLAYSSM_MAMBA2>(dk, a, s);
}

__global__ void __launch_bounds__(256) eager_accept_kernel(int32_t* slot, const int32_t* acc, int B,
                                                           int T) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  int ab = acc[b];
  ab = ab < 0 ? 0 : (ab > T ? T : ab);
  int s0 = slot[b];
  if (s0 < 0 || s0 > T) s0 = 0;
  slot[b] = (s0 + ab) % (T + 1);
}

hipError_t launch_eager_accept(int32_t* slot, const int32_t* acc, int B, int T, hipStream_t s) {
  hipLaunchKernelGGL(eager_accept_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, slot,
                     acc, B, T);
  return hipGetLastError();
}

}  // namespace rs
