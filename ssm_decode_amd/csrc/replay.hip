// Replay kernel of libreplayssm: standard decode, output-only draft
// verification and the checkpoint fold, for Mamba-2 and Gated DeltaNet heads.
//
// One workgroup owns one (sequence b, head) pair and one wavefront owns one
// 16-row tile of the head's state (dv / 16 wavefronts). A call:
//
//  1. streams the head's checkpoint from HBM into registers (fp32, or the bf16
//     copy on non-fold steps in the two-precision mode), and stages the records
//     of the ring (alpha, k, v / u) plus the drafts' q in LDS;
//  2. decides the route per sequence: fold when h + T > L (flowchart in
//     "ReplaySSM: Cache SSM Inputs, Not State", How it works); the flush call
//     folds whenever h > 0;
//  3. fold route: S <- Gamma_h S + V diag(gamma) K^T over the h committed
//     records as MFMA rank-4 steps whose accumulators are the checkpoint
//     registers themselves, then writes the fp32 and/or bf16 checkpoint; the
//     drafts are then replayed on top of the new state held in registers (the
//     author's reply on the flush route: the state from one V K^T product, the
//     output by multiplying it with q);
//  4. replay route (no state write): o_i = Gamma_i S q_i
//     + sum_r gamma_{r,i} (k_r . q_i) v_r over the buffered records r up to
//     draft i ("How it works": Standard decoding and Speculative decoding);
//     the k_r . q_i products are wavefront reductions, the decay products
//     gamma are running products of alpha (no logarithms, so alpha = 0 is
//     exact);
//  5. GDN: u_i = beta_i (v_i - alpha_i S_{i-1} k_i) with S_{i-1} k_i rebuilt
//     from S k_i and the buffer ("How it works": Gated DeltaNet), sequential
//     over the drafts, and stored in place of v_i;
//  6. the last workgroup of the sequence to finish advances its pointers.
#include "device.hpp"

namespace rs {

template <int KIND, int NT, int TMAX>
__global__ void __launch_bounds__(1024) replay_kernel(const ReplayArgs a) {
  constexpr int DK = NT * 16;
  constexpr int LPR = DK / 4;       // lanes per k row in the dot phase (float4 each)
  constexpr int RPI = kWave / LPR;  // k rows per wavefront pass
  constexpr bool GDN = (KIND == REPLAYSSM_GDN);
  extern __shared__ f32x4 smem_v4[];
  float* sm = reinterpret_cast<float*>(smem_v4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthr = blockDim.x;
  const int W = nthr >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int H = a.H, C = a.C, dv = a.dv;
  const int b = blockIdx.x / H;
  const int hd = blockIdx.x - b * H;
  const int64_t bh = (int64_t)b * H + hd;
  const int prow = wave * 16 + col;  // the state row this lane owns
  const ReplayLds lds(C, DK, dv, TMAX);

  const int head = a.head[b];
  const int hc = a.h[b];
  const int pend = a.p[b];
  const int mode = a.mode;
  const int T = (mode == kModeFlush) ? 0 : a.T;
  // pointers outside their invariant ranges would address outside the ring
  const bool corrupt = head < 0 || head >= C || hc < 0 || hc > a.L || pend < 0 || pend > C - a.L;
  const bool bad = corrupt || ((mode != kModeFlush) && (pend != T));
  const bool fold = !bad && ((mode == kModeFlush) ? (hc > 0) : (hc + T > a.L));
  const bool work = !bad && (mode != kModeFlush || fold);
  const bool outputs = work && (mode != kModeFlush);
  const int R = hc + T;          // staged records: committed [0, hc), drafts [hc, hc + T)
  const int r0 = fold ? hc : 0;  // first record replayed on top of the checkpoint
  const int prec = a.precision;
  const bool read_lp =
      (prec == REPLAYSSM_BF16_SHARED) || (prec == REPLAYSSM_FP32_HP_BF16_LP && !fold);

  // ---- 1. checkpoint into registers, records into LDS -----------------------
  f32x4 S[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (work) {
    const int64_t hoff = bh * (int64_t)(dv * DK);
    if (!read_lp) {
      const float* src = a.hp + hoff + (int64_t)(wave * NT) * 256 + lane * 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S[nt] = ld4(src + nt * 256);
    } else if constexpr (NT >= 2) {
      const uint4* src = reinterpret_cast<const uint4*>(a.lp + hoff) + (wave * NT / 2) * 64 + lane;
#pragma unroll
      for (int m = 0; m < NT / 2; ++m) unpack_lp_chunk(src[m * 64], S[2 * m], S[2 * m + 1]);
    }

    const float* rk = a.ring_k + bh * (int64_t)C * DK;
    const float* rv = a.ring_v + bh * (int64_t)C * dv;
    {  // k rows: LPR threads per row
      const int r_in = tid / LPR, c4 = tid % LPR;
      for (int r = r_in; r < R; r += nthr / LPR) {
        int slot = head + r;
        if (slot >= C) slot -= C;
        st4(sm + lds.k + r * lds.dks + 4 * c4, ld4(rk + slot * DK + 4 * c4));
      }
    }
    {  // v rows: dv / 4 threads per row (nthr = 16 * dv / 4)
      const int dv4 = dv >> 2;
      const int r_in = tid / dv4, c4 = tid - (tid / dv4) * dv4;
      for (int r = r_in; r < R; r += 16) {
        int slot = head + r;
        if (slot >= C) slot -= C;
        st4(sm + lds.v + r * lds.dvs + 4 * c4, ld4(rv + slot * dv + 4 * c4));
      }
    }
    for (int r = tid; r < R; r += nthr) {
      int slot = head + r;
      if (slot >= C) slot -= C;
      sm[lds.alpha + r] = a.ring_alpha[bh * C + slot];
      if (GDN && r >= hc) sm[lds.beta + (r - hc)] = a.ring_beta[bh * C + slot];
    }
    for (int idx = tid; idx < TMAX * LPR; idx += nthr) {
      const int i = idx / LPR, c4 = idx % LPR;
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < T) x = ld4(a.q + (((int64_t)b * T + i) * H + hd) * DK + 4 * c4);
      st4(sm + lds.q + i * DK + 4 * c4, x);
    }
  }
  __syncthreads();

  // ---- 2. decay products and record dot products -----------------------------
  if (outputs) {
    // Row r + 1 of gq / gk, for r in [r0 - 1, R): gq[.][i] = prod of alpha over
    // records (r, hc + i] (decay of record r at draft i), gk[.][i] the same over
    // (r, hc + i - 1] (the state just before draft i). Row r0 (r = r0 - 1) thus
    // holds the checkpoint's factors Gamma_i and Gamma_{i-1}. Entries for
    // records that come after the draft stay zero.
    for (int t = tid; t < R - r0 + 1; t += nthr) {
      const int r = r0 - 1 + t;
      float* gq = sm + lds.gq + (r + 1) * TMAX;
      float* gk = sm + lds.gk + (r + 1) * TMAX;
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        gq[i] = 0.f;
        gk[i] = 0.f;
      }
      float prod = 1.f;
      for (int rr = r + 1; rr < R; ++rr) {
        const int i = rr - hc;
        if (i >= 0) gk[i] = prod;
        prod *= sm[lds.alpha + rr];
        if (i >= 0) gq[i] = prod;
      }
      if (r >= hc) gq[r - hc] = 1.f;
    }
  }
  if (fold) {
    // gf[t] = prod of alpha over committed records [t, hc): gf[0] = Gamma_h
    // scales the checkpoint, gf[j + 1] weighs record j in the fold.
    for (int t = tid; t <= hc; t += nthr) {
      float prod = 1.f;
      for (int rr = t; rr < hc; ++rr) prod *= sm[lds.alpha + rr];
      sm[lds.gf + t] = prod;
    }
  }
  if (outputs) {
    const int sub = lane / LPR, li = lane % LPR;
    f32x4 qf[TMAX], kf[TMAX];
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
      qf[i] = ld4(sm + lds.q + i * DK + 4 * li);
      kf[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (GDN && i < T) kf[i] = ld4(sm + lds.k + (hc + i) * lds.dks + 4 * li);
    }
    for (int base = r0 + wave * RPI; base < R; base += W * RPI) {
      const int r = base + sub;
      const bool valid = r < R;
      f32x4 kr = f32x4{0.f, 0.f, 0.f, 0.f};
      if (valid) kr = ld4(sm + lds.k + r * lds.dks + 4 * li);
      float dq[TMAX], dkk[TMAX];
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        dq[i] = sum_width<LPR>(dot4(kr, qf[i]));
        dkk[i] = GDN ? sum_width<LPR>(dot4(kr, kf[i])) : 0.f;
      }
      if (valid && li == 0) {
#pragma unroll
        for (int i = 0; i < TMAX; ++i) {
          sm[lds.cq + r * TMAX + i] = dq[i];
          if (GDN) sm[lds.ck + r * TMAX + i] = dkk[i];
        }
      }
    }
  }
  __syncthreads();

  // ---- 3. fold: S <- Gamma_h S + sum_j gamma_j v_j k_j^T on MFMA ------------
  if (fold) {
    const float G = sm[lds.gf];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) S[nt] *= G;
    // MFMA 16x16x4: A[m][kk] = k_j[16 nt + m], B[kk][n] = gamma_j v_j[16 wave + n],
    // j = 4 kc + kk; lane l supplies A[l & 15][l >> 4] and B[l >> 4][l & 15].
    const int nkc = (hc + 3) >> 2;
    for (int kc = 0; kc < nkc; ++kc) {
      const int j = 4 * kc + g;
      const bool vj = j < hc;
      const float bval = vj ? sm[lds.gf + j + 1] * sm[lds.v + j * lds.dvs + prow] : 0.f;
      const float* krow = sm + lds.k + (vj ? j : 0) * lds.dks + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float aval = vj ? krow[nt * 16] : 0.f;
        S[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bval, S[nt], 0, 0, 0);
      }
    }
    const int64_t hoff = bh * (int64_t)(dv * DK);
    if (prec != REPLAYSSM_BF16_SHARED) {
      float* dst = a.hp + hoff + (int64_t)(wave * NT) * 256 + lane * 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st4(dst + nt * 256, S[nt]);
    }
    if constexpr (NT >= 2) {
      if (prec != REPLAYSSM_FP32) {
        uint4* dst = reinterpret_cast<uint4*>(a.lp + hoff) + (wave * NT / 2) * 64 + lane;
#pragma unroll
        for (int m = 0; m < NT / 2; ++m) {
          const uint4 x = pack_lp_chunk(S[2 * m], S[2 * m + 1]);
          dst[m * 64] = x;
          if (prec == REPLAYSSM_BF16_SHARED) unpack_lp_chunk(x, S[2 * m], S[2 * m + 1]);
        }
      }
    }
  }

  // ---- 4/5. outputs of the drafts ---------------------------------------------
  if (outputs) {
    float yq[TMAX], yk[TMAX];
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
      yq[i] = 0.f;
      yk[i] = 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        if (i < T) {
          yq[i] += dot4(S[nt], ld4(sm + lds.q + i * DK + nt * 16 + 4 * g));
          if (GDN) yk[i] += dot4(S[nt], ld4(sm + lds.k + (hc + i) * lds.dks + nt * 16 + 4 * g));
        }
      }
    }
    const float* gq = sm + lds.gq;
    const float* gk = sm + lds.gk;
    const float* cq = sm + lds.cq;
    const float* ck = sm + lds.ck;
    const float* sv = sm + lds.v + prow;
    if constexpr (!GDN) {
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        if (i < T) {
          float acc = gq[r0 * TMAX + i] * yq[i];
          for (int r = r0 + g; r <= hc + i; r += 4)
            acc += gq[(r + 1) * TMAX + i] * cq[r * TMAX + i] * sv[r * lds.dvs];
          acc = sum_groups(acc);
          if (g == 0) a.out[(((int64_t)b * T + i) * H + hd) * dv + prow] = acc;
        }
      }
    } else {
      // committed records in parallel over the four lane groups
      float wc[TMAX], oc[TMAX];
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        wc[i] = 0.f;
        oc[i] = 0.f;
        if (i < T) {
          wc[i] = gk[r0 * TMAX + i] * yk[i];
          oc[i] = gq[r0 * TMAX + i] * yq[i];
          for (int r = r0 + g; r < hc; r += 4) {
            const float u = sv[r * lds.dvs];
            wc[i] += gk[(r + 1) * TMAX + i] * ck[r * TMAX + i] * u;
            oc[i] += gq[(r + 1) * TMAX + i] * cq[r * TMAX + i] * u;
          }
          wc[i] = sum_groups(wc[i]);
          oc[i] = sum_groups(oc[i]);
        }
      }
      // drafts in order: u_i needs the corrections of the drafts before it
      float ud[TMAX];
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        ud[i] = 0.f;
        if (i < T) {
          float w = wc[i];
#pragma unroll
          for (int d = 0; d < i; ++d) w += gk[(hc + d + 1) * TMAX + i] * ck[(hc + d) * TMAX + i] * ud[d];
          const float al = sm[lds.alpha + hc + i];
          const float be = sm[lds.beta + i];
          ud[i] = be * (sv[(hc + i) * lds.dvs] - al * w);
          float o = oc[i];
#pragma unroll
          for (int d = 0; d <= i; ++d) o += gq[(hc + d + 1) * TMAX + i] * cq[(hc + d) * TMAX + i] * ud[d];
          if (g == 0) {
            a.out[(((int64_t)b * T + i) * H + hd) * dv + prow] = o;
            int slot = head + hc + i;
            if (slot >= C) slot -= C;
            a.ring_v[(bh * C + slot) * dv + prow] = ud[i];
          }
        }
      }
    }
  }

  // ---- 6. pointers ------------------------------------------------------------
  __syncthreads();
  if (tid == 0 && arrive_last(a.arrive, b, H)) {
    if (bad) {
      atomicOr(a.err, corrupt ? REPLAYSSM_DEVERR_CORRUPT : REPLAYSSM_DEVERR_PENDING);
    } else {
      int nhead = head, nh = hc;
      int64_t nf = a.folded[b];
      if (fold) {
        nhead = head + hc;
        if (nhead >= C) nhead -= C;
        nf += hc;
        nh = 0;
      }
      if (mode == kModeDecode) {
        nh += 1;
        a.p[b] = 0;
      }
      a.head[b] = nhead;
      a.h[b] = nh;
      a.folded[b] = nf;
    }
  }
}

template <int KIND, int NT, int TMAX>
static hipError_t launch_t(const ReplayArgs& a, hipStream_t s) {
  const ReplayLds lds(a.C, NT * 16, a.dv, TMAX);
  const dim3 grid((unsigned)(a.B * a.H));
  const dim3 block((unsigned)(a.dv / 16 * kWave));
  hipLaunchKernelGGL((replay_kernel<KIND, NT, TMAX>), grid, block, (size_t)lds.total * 4, s, a);
  return hipGetLastError();
}

template <int KIND, int NT>
static hipError_t launch_nt(int tmax, const ReplayArgs& a, hipStream_t s) {
  switch (tmax) {
    case 1: return launch_t<KIND, NT, 1>(a, s);
    case 4: return launch_t<KIND, NT, 4>(a, s);
    case 8: return launch_t<KIND, NT, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int KIND>
static hipError_t launch_kind(int dk, int tmax, const ReplayArgs& a, hipStream_t s) {
  switch (dk) {
    case 16: return launch_nt<KIND, 1>(tmax, a, s);
    case 32: return launch_nt<KIND, 2>(tmax, a, s);
    case 64: return launch_nt<KIND, 4>(tmax, a, s);
    case 128: return launch_nt<KIND, 8>(tmax, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_replay(int kind, int dk, int tmax, const ReplayArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  return kind == REPLAYSSM_GDN ? launch_kind<REPLAYSSM_GDN>(dk, tmax, a, s)
                               : launch_kind<REPLAYSSM_MAMBA2>(dk, tmax, a, s);
}

}  // namespace rs
