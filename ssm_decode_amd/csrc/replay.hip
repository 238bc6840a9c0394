// Replay kernel of libreplayssm: standard decode, output-only draft
// verification and the checkpoint fold, for Mamba-2, Gated DeltaNet and Kimi
// Delta Attention (per-channel gate) heads.
//
// The work items are (sequence b, head) pairs. A workgroup holds one item at a
// time, one wavefront per 16-row tile of the head's state (dv / 16
// wavefronts), and walks its items with the stride of the grid (persistent
// workgroups). For one item:
//
//  1. its checkpoint sits in registers (fp32, or the bf16 copy on non-fold
//     steps in the two-precision mode) and its ring records (alpha, k, v / u)
//     plus the drafts' q go to LDS; both were requested while the workgroup
//     worked on its previous item;
//  2. the route is decided per sequence: fold when h + T > L (flowchart in
//     "ReplaySSM: Cache SSM Inputs, Not State", How it works); the flush call
//     folds whenever h > 0;
//  3. fold route: S <- Gamma_h S + V diag(gamma) K^T over the h committed
//     records as MFMA rank-4 steps whose accumulators are the checkpoint
//     registers themselves, then the fp32 and/or bf16 checkpoint is written;
//     the drafts are then replayed on top of the new state held in registers
//     (the author's reply on the flush route: the state from one V K^T
//     product, the output by multiplying it with q);
//  4. replay route (no state write): o_i = Gamma_i S q_i
//     + sum_r gamma_{r,i} (k_r . q_i) v_r over the buffered records r up to
//     draft i ("How it works": Standard decoding and Speculative decoding);
//     the k_r . q_i products are wavefront reductions, the decay products
//     gamma are products of alpha (suffix scans, no logarithms, so alpha = 0 is
//     exact);
//  5. GDN: u_i = beta_i (v_i - alpha_i S_{i-1} k_i) with S_{i-1} k_i rebuilt
//     from S k_i and the buffer ("How it works": Gated DeltaNet), sequential
//     over the drafts, and stored in place of v_i; KDA: the same with a gate
//     vector per record, whose products are applied to the staged keys and
//     queries per channel instead of being tabulated per record;
//  6. the pointers are only read while items run; the last workgroup of the
//     grid to finish advances them for every sequence.
//
// Pipelining: right after step 1 the workgroup requests the next item's ring
// records (into registers), and as soon as this item's mat-vecs have consumed
// S, the next item's checkpoint (into S, in the precision that item's route
// reads). Both stream in while this item computes. Vector memory operations
// complete in order and the compiler waits on them by count, taking the
// smallest count over every control-flow path; so every path through an item
// issues the same record loads in the same order (a load that has nothing to
// fetch reads one fixed location instead of being skipped) and makes the
// checkpoint request at one program point: the next item then waits for its
// records without waiting for its checkpoint, and for its checkpoint without
// waiting for the records requested after it.
#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "route.hpp"

namespace rs {

// Which checkpoint copy an item reads: the bf16 one in the shared-bf16 mode,
// and on the non-fold steps of the two-precision mode; fp32 otherwise.
__device__ __forceinline__ bool reads_lp(int precision, bool fold) {
  return precision == REPLAYSSM_BF16_SHARED || (precision == REPLAYSSM_FP32_HP_BF16_LP && !fold);
}

// GDN with the two-precision checkpoint: a fold recomputes the folded records'
// corrections from the fp32 checkpoint and their raw v.
template <int KIND>
__device__ __forceinline__ bool exact_fold(const Route& rt) {
  return KIND == kKindGdnExact && rt.fold;
}

// Requests the checkpoint copy of `item` into S: the fp32 tiles, or the bf16
// copy's raw 16-byte chunks in S[0, NT/2) (widened in place when used), with
// computed addresses and no branch; with valid false (no item, or an item with
// nothing to do) every load reads the array's first bytes. (The bf16 form issues
// half the loads of the fp32 one; padding it to the same count, which keeps the
// compiler's waits after it exact, measured slower than the waits it saves.)
template <int NT>
__device__ __forceinline__ void prefetch_ckpt(const ReplayArgs& a, int item, bool fold, bool valid, int wave,
                                              int lane, f32x4 (&S)[NT]) {
  const bool lp = reads_lp(a.precision, fold);
  const char* base = lp ? reinterpret_cast<const char*>(a.lp) : reinterpret_cast<const char*>(a.hp);
  const int64_t head_bytes = (int64_t)a.dv * NT * 16 * (lp ? 2 : 4);
  const int first_chunk = lp ? wave * (NT / 2) : wave * NT;  // 1 KiB chunks: 64 lanes x 16 bytes
  const int64_t start = valid ? (int64_t)item * head_bytes + (int64_t)first_chunk * 1024 + lane * 16 : 0;
  const int step = valid ? 1024 : 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (lp && nt >= NT / 2) continue;
    const char* src = base + start + nt * step;
    S[nt] = __builtin_bit_cast(f32x4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src)));
  }
}

// One item's ring rows while they are in flight: up to K k-row and V v-row
// passes per thread (a pass is nthr / (dk / 4) k rows or nthr / (dv / 4) v rows), the
// thread's float4 of the drafts' q, and its alpha / beta. Rows beyond the
// passes go through the tail loop of store_records, which waits for each row.
// With dk = 128 and dv >= 64 two k passes and one v pass cover 16 rows (two v
// passes with two tiles per wavefront, whose workgroup is half as large). (Every
// pass is issued whether or not its rows exist, which keeps the compiler's
// memory waits exact but costs a request per pass: three k and two v passes
// for the verify kernels measured slower than the tail loop they save.)
template <int TMAX, int VP = 1>
struct RecRegs {
  static constexpr int K = 2, V = VP;
  f32x4 kb[K], vb[V], qv;
  f32x4 ab[K];  // KDA: the gate rows, staged like the k rows (unused by the other kinds)
  float al, be;
};

// Where a thread's share of the ring rows lies (k rows: LPR threads per row;
// v rows: dv / 4 threads per row, vstep rows per pass: 16 with one wavefront per
// 16-row tile, 8 with two tiles per wavefront).
struct StageMap {
  int kstep, rk0, ck, rv0, cv, vstep;
  __device__ __forceinline__ StageMap(int tid, int nthr, int lpr, int dv) {
    kstep = nthr / lpr;
    rk0 = tid / lpr;
    ck = tid % lpr;
    const int dv4 = dv >> 2;
    rv0 = tid / dv4;
    cv = tid - rv0 * dv4;
    vstep = nthr / dv4;
  }
};

// A work item: its index and its (sequence, head), stepped along with the
// index so that no item divides by H.
struct Item {
  int id, b, hd;
};

// Source rows of one item: committed records from the ring; the drafts from
// the ring too, or, in a fused call, straight from the caller's inputs.
struct RowSrc {
  const float* rk;   // ring k rows of the head
  const float* rv;   // ring v rows
  const float* rvraw;  // raw v rows (GDN with the two-precision checkpoint), else rv
  const float* ik;   // input k of draft 0 (fused), stride H * dk per draft
  const float* iv;   // input v of draft 0 (fused), stride H * dv per draft
  int64_t ia;        // index of draft 0 in the alpha / beta inputs, stride H per draft
  int64_t bhC;       // first ring slot index of the head
};

template <int NT>
__device__ __forceinline__ RowSrc row_src(const ReplayArgs& a, const Item& it, int T) {
  constexpr int DK = NT * 16;
  const int H = a.H, C = a.C, dv = a.dv;
  const int b = it.b, hd = it.hd;
  const int64_t bh = (int64_t)b * H + hd;
  RowSrc s;
  s.rk = a.ring_k + bh * (int64_t)C * DK;
  s.rv = a.ring_v + bh * (int64_t)C * dv;
  s.rvraw = a.ring_vraw ? a.ring_vraw + bh * (int64_t)C * dv : s.rv;
  s.ia = (int64_t)b * T * H + hd;
  s.ik = a.in_k + s.ia * DK;
  s.iv = a.in_v + s.ia * dv;
  s.bhC = bh * C;
  return s;
}

template <int KIND, int NT, int TMAX, bool FUSED, int RT>
__device__ __forceinline__ void load_records(const ReplayArgs& a, const Item& item, const SeqPtr& p,
                                             const Route& rt, bool valid, int tid, const StageMap& m,
                                             RecRegs<TMAX, RT>& rr) {
  constexpr int kRecK = RecRegs<TMAX, RT>::K, kRecV = RecRegs<TMAX, RT>::V;
  constexpr int DK = NT * 16;
  // Every load is issued; one with nothing to fetch reads the first element of a
  // ring array (always allocated: q and the inputs are NULL in a flush call).
  const bool ok = valid && rt.work;
  const int H = a.H, C = a.C, dv = a.dv, T = ok ? rt.T : 0, R = ok ? rt.R : 0;
  const Item it = ok ? item : Item{0, 0, 0};
  const int b = it.b, hd = it.hd;
  const RowSrc s = row_src<NT>(a, it, T);
  constexpr bool fused = FUSED;
#pragma unroll
  for (int j = 0; j < kRecK; ++j) {
    const int r = m.rk0 + j * m.kstep;
    const float* src = (fused && r >= p.h) ? s.ik + (int64_t)(r - p.h) * H * DK + 4 * m.ck
                                           : s.rk + ring_slot(p.head, r, C) * DK + 4 * m.ck;
    rr.kb[j] = ld4(r < R ? src : a.ring_k);
    if constexpr (KIND == REPLAYSSM_KDA) {
      const float* asrc = (fused && r >= p.h) ? a.in_alpha + (s.ia + (int64_t)(r - p.h) * H) * DK + 4 * m.ck
                                              : a.ring_alpha + (s.bhC + ring_slot(p.head, r, C)) * DK + 4 * m.ck;
      rr.ab[j] = ld4(r < R ? asrc : a.ring_alpha);
    }
  }
  // a fold with exact corrections stages the committed records' raw v instead of
  // their stored corrections
  const bool raw = exact_fold<KIND>(rt);
#pragma unroll
  for (int j = 0; j < kRecV; ++j) {
    const int r = m.rv0 + j * m.vstep;
    const float* src = (fused && r >= p.h) ? s.iv + (int64_t)(r - p.h) * H * dv + 4 * m.cv
                                           : (raw && r < p.h ? s.rvraw : s.rv) + ring_slot(p.head, r, C) * dv + 4 * m.cv;
    rr.vb[j] = ld4(r < R ? src : a.ring_v);
  }
  // q is read once per call: non-temporal, like the checkpoint stream
  rr.qv = ld4_stream(m.rk0 < T ? a.q + (((int64_t)b * T + m.rk0) * H + hd) * DK + 4 * m.ck : a.ring_k);
  if constexpr (KIND != REPLAYSSM_KDA) {
    const float* src = (fused && tid >= p.h) ? a.in_alpha + s.ia + (int64_t)(tid - p.h) * H
                                             : a.ring_alpha + s.bhC + ring_slot(p.head, tid, C);
    rr.al = *(tid < R ? src : a.ring_alpha);
  }
  if constexpr (kind_gdn(KIND)) {
    const float* src = (fused && tid >= p.h) ? a.in_beta + s.ia + (int64_t)(tid - p.h) * H
                                             : a.ring_beta + s.bhC + ring_slot(p.head, tid, C);
    rr.be = *((tid < R && (tid >= p.h || raw)) ? src : a.ring_beta);
  }
}

// The item's rows into LDS: from the registers, and the rows beyond the
// register passes straight from HBM.
// A fused call also writes the drafts' records into their ring slots (k,
// alpha, and v for Mamba-2 / beta for GDN, whose u replaces v later).
template <int KIND, int NT, int TMAX, bool FUSED, int RT>
__device__ __forceinline__ void store_records(const ReplayArgs& a, float* sm, const ReplayLds& lds,
                                              const Item& item, const SeqPtr& p, const Route& rt, int tid,
                                              int nthr, const StageMap& m, const RecRegs<TMAX, RT>& rr) {
  constexpr int kRecK = RecRegs<TMAX, RT>::K, kRecV = RecRegs<TMAX, RT>::V;
  constexpr int DK = NT * 16;
  constexpr bool GDN = kind_gdn(KIND);
  const bool raw = exact_fold<KIND>(rt);
  const int H = a.H, C = a.C, dv = a.dv, T = rt.T, R = rt.R;
  const int b = item.b, hd = item.hd;
  const RowSrc s = row_src<NT>(a, item, T);
  constexpr bool fused = FUSED;
  float* wk = a.ring_k + (s.rk - a.ring_k);
  float* wv = a.ring_v + (s.rv - a.ring_v);
  // the register rows first: their registers are then free for the tail loads
#pragma unroll
  for (int j = 0; j < kRecK; ++j) {
    const int r = m.rk0 + j * m.kstep;
    if (r < R) {
      st4(sm + lds.k + r * lds.dks + 4 * m.ck, rr.kb[j]);
      if (fused && r >= p.h) st4(wk + ring_slot(p.head, r, C) * DK + 4 * m.ck, rr.kb[j]);
      if constexpr (KIND == REPLAYSSM_KDA) {
        st4(sm + lds.alpha + r * lds.dks + 4 * m.ck, rr.ab[j]);
        if (fused && r >= p.h) st4(a.ring_alpha + (s.bhC + ring_slot(p.head, r, C)) * DK + 4 * m.ck, rr.ab[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kRecV; ++j) {
    const int r = m.rv0 + j * m.vstep;
    if (r < R) {
      st4(sm + lds.v + r * lds.dvs + 4 * m.cv, rr.vb[j]);
      if (!GDN && fused && r >= p.h) st4(wv + ring_slot(p.head, r, C) * dv + 4 * m.cv, rr.vb[j]);
      if (GDN && fused && r >= p.h && a.ring_vraw)
        st4(a.ring_vraw + (s.rv - a.ring_v) + ring_slot(p.head, r, C) * dv + 4 * m.cv, rr.vb[j]);
    }
  }
  if (m.rk0 < T) st4(sm + lds.q + m.rk0 * DK + 4 * m.ck, rr.qv);
  for (int i = (m.rk0 < T ? m.rk0 + m.kstep : m.rk0); i < TMAX; i += m.kstep)
    if (i >= T) st4(sm + lds.q + i * DK + 4 * m.ck, f32x4{0.f, 0.f, 0.f, 0.f});  // rows of absent drafts
  if (tid < R) {
    if constexpr (KIND != REPLAYSSM_KDA) {
      sm[lds.alpha + tid] = rr.al;
      if (fused && tid >= p.h) a.ring_alpha[s.bhC + ring_slot(p.head, tid, C)] = rr.al;
    }
    if (GDN && (tid >= p.h || raw)) {
      sm[lds.beta + tid] = rr.be;
      if (fused && tid >= p.h) a.ring_beta[s.bhC + ring_slot(p.head, tid, C)] = rr.be;
    }
  }
  // k rows past the register passes: kTail rows' loads issued together, then
  // their stores (one memory round trip per group instead of one per row; no
  // load of a group reads a slot that a store of the same group writes)
  constexpr int kTail = KIND == REPLAYSSM_KDA ? 1 : 4;
  for (int r0 = m.rk0 + kRecK * m.kstep; r0 < R; r0 += kTail * m.kstep) {
    f32x4 x[kTail], y[kTail];
#pragma unroll
    for (int u = 0; u < kTail; ++u) {
      const int r = r0 + u * m.kstep;
      const bool in = fused && r >= p.h;
      const int slot = ring_slot(p.head, r, C);
      x[u] = ld4(r >= R ? a.ring_k : in ? s.ik + (int64_t)(r - p.h) * H * DK + 4 * m.ck : s.rk + slot * DK + 4 * m.ck);
      if constexpr (KIND == REPLAYSSM_KDA)
        y[u] = ld4(r >= R ? a.ring_alpha
                          : in ? a.in_alpha + (s.ia + (int64_t)(r - p.h) * H) * DK + 4 * m.ck
                               : a.ring_alpha + (s.bhC + slot) * DK + 4 * m.ck);
    }
#pragma unroll
    for (int u = 0; u < kTail; ++u) {
      const int r = r0 + u * m.kstep;
      if (r < R) {
        const bool in = fused && r >= p.h;
        const int slot = ring_slot(p.head, r, C);
        st4(sm + lds.k + r * lds.dks + 4 * m.ck, x[u]);
        if (in) st4(wk + slot * DK + 4 * m.ck, x[u]);
        if constexpr (KIND == REPLAYSSM_KDA) {
          st4(sm + lds.alpha + r * lds.dks + 4 * m.ck, y[u]);
          if (in) st4(a.ring_alpha + (s.bhC + slot) * DK + 4 * m.ck, y[u]);
        }
      }
    }
  }
  for (int r = m.rv0 + kRecV * m.vstep; r < R; r += m.vstep) {
    const int slot = ring_slot(p.head, r, C);
    const bool in = fused && r >= p.h;
    const f32x4 x = ld4(in ? s.iv + (int64_t)(r - p.h) * H * dv + 4 * m.cv
                           : (raw && r < p.h ? s.rvraw : s.rv) + slot * dv + 4 * m.cv);
    st4(sm + lds.v + r * lds.dvs + 4 * m.cv, x);
    if (in && !GDN) st4(wv + slot * dv + 4 * m.cv, x);
    if (in && GDN && a.ring_vraw) st4(a.ring_vraw + (s.rv - a.ring_v) + slot * dv + 4 * m.cv, x);
  }
  for (int i = m.rk0 + m.kstep; i < T; i += m.kstep)
    st4(sm + lds.q + i * DK + 4 * m.ck, ld4_stream(a.q + (((int64_t)b * T + i) * H + hd) * DK + 4 * m.ck));
  for (int r = tid + nthr; r < R; r += nthr) {
    const int slot = ring_slot(p.head, r, C);
    const bool in = fused && r >= p.h;
    if constexpr (KIND != REPLAYSSM_KDA) {
      const float al = in ? a.in_alpha[s.ia + (int64_t)(r - p.h) * H] : a.ring_alpha[s.bhC + slot];
      sm[lds.alpha + r] = al;
      if (in) a.ring_alpha[s.bhC + slot] = al;
    }
    if (GDN && (r >= p.h || raw)) {
      const float be = in ? a.in_beta[s.ia + (int64_t)(r - p.h) * H] : a.ring_beta[s.bhC + slot];
      sm[lds.beta + r] = be;
      if (in) a.ring_beta[s.bhC + slot] = be;
    }
  }
}

// Whether the mat-vecs run on the matrix cores (matvec_mfma in replay_item): the delta-rule
// kinds with 4 or 8 drafts, whose 8 or 16 right-hand vectors fill half or all of the operand.
// (Timed against the vector form on MI355X: equal within run-to-run spread for every kind.)
template <int KIND, int TMAX>
constexpr bool kMfmaMatvec = kind_gdn(KIND) && TMAX >= 4;

// One item. On entry S holds (or is loading) the checkpoint copy the item's
// route reads, and rr its ring rows; both were requested during the previous
// item. On return rr holds (or is loading) the rows of `next` and S its
// checkpoint copy. Ends with a workgroup barrier after its last LDS read.
template <int KIND, int NT, int TMAX, bool FUSED, int RT>
__device__ __forceinline__ void replay_item(const ReplayArgs& a, float* sm, const ReplayLds& lds,
                                            const StageMap& map0, const Item it, const SeqPtr ptr, const Route rt,
                                            f32x4 (&S)[RT * NT], RecRegs<TMAX, RT>& rr, const Item nit,
                                            const SeqPtr nptr, const Route nrt) {
  constexpr int DK = NT * 16;
  // Dot phase: each lane takes CPL float4 chunks of a k row (chunks li and
  // li + LPR), so LPR lanes share a row and a wavefront pass covers RPI rows.
  // Two chunks per lane halve the passes and the reduction tree loses a level;
  // the verify kernels with 8 drafts keep one chunk (their registers are full).
  constexpr int CPL = (KIND != REPLAYSSM_KDA && TMAX <= 4 && DK >= 32) ? 2 : 1;
  constexpr int LPR = DK / (4 * CPL);
  constexpr int RPI = kWave / LPR;
  constexpr bool GDN = kind_gdn(KIND);
  constexpr bool KDA = KIND == REPLAYSSM_KDA;

  // The thread index is laundered per item: without it the compiler hoists
  // every thread-derived address out of the item loop and keeps them all live
  // across it, which doubles the register footprint and halves occupancy.
  int tid = threadIdx.x;
  __asm__ volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthr = blockDim.x;
  const int W = nthr >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int H = a.H, C = a.C, dv = a.dv;
  const int b = it.b;
  const int hd = it.hd;
  const int64_t bh = (int64_t)b * H + hd;
  // RT 16-row tiles per wavefront: the lane owns state rows prow + 16 tl, tl < RT
  const int prow = wave * RT * 16 + col;
  using Tile = f32x4[NT];
  auto tile = [&](int tl) -> Tile& { return *reinterpret_cast<Tile*>(&S[tl * NT]); };
  // (the staging map is computed once per workgroup and laundered like tid)
  StageMap map = map0;
  __asm__ volatile("" : "+v"(map.rk0), "+v"(map.ck), "+v"(map.rv0), "+v"(map.cv));

  const int mode = a.mode;
  const int prec = a.precision;
  const int64_t hoff = bh * (int64_t)(dv * DK);

  // The pointers were read before this item started (in the workgroup's
  // batch read); they are written only after every workgroup is done.
  const int head = ptr.head;
  const int hc = ptr.h;
  const int T = rt.T;
  const bool corrupt = rt.corrupt, bad = rt.bad, fold = rt.fold, work = rt.work, outputs = rt.outputs;
  const int R = rt.R, r0 = rt.r0;

  // ---- 1. records (the checkpoint copy is already in flight) --------------------
  if (work) store_records<KIND, NT, TMAX, FUSED, RT>(a, sm, lds, it, ptr, rt, tid, nthr, map, rr);
  __syncthreads();

  // ---- the next item's ring rows: requested now, waited for by the next item
  const bool more = nit.id < a.B * a.H;
  load_records<KIND, NT, TMAX, FUSED, RT>(a, nit, nptr, nrt, more, tid, map, rr);

  // ---- KDA: the gate products, per channel (a thread per channel and job) ------
  // With per-channel gates the state after records [0, m] is
  //   S_m = S Diag(prod of a_r, r <= m) + sum_r u_r (k_r * prod of a_s, r < s <= m)^T,
  // so the products go onto the vectors instead of into decay tables:
  //  - committed records: k_j <- k_j * prod of a over (j, hc) in place, and
  //    pf = prod of a over [0, hc), so that S_h = S Diag(pf) + sum_j u_j k_j^T;
  //  - drafts: Gamma_i = prod of a over [hc, hc + i], qg_i = Gamma_i * q_i and
  //    kg_i = Gamma_i * k_{hc+i}: o_i needs S_h qg_i and u_i needs S_h kg_i
  //    (the draft's own gate sits in kg_i, as S_{m-1} (a_m * k_m) requires);
  //  - draft-to-draft terms take the gates between the two drafts, applied
  //    in the dot-product pass.
  if constexpr (KDA) {
    if (work) {
      for (int u = tid; u < 2 * DK; u += nthr) {
        if (u < DK) {
          const int n = u;
          float s = 1.f;
          for (int j = hc - 1; j >= 0; --j) {
            sm[lds.k + j * lds.dks + n] *= s;
            s *= sm[lds.alpha + j * lds.dks + n];
          }
          sm[lds.pf + n] = s;
        } else {
          const int n = u - DK;
          float gm = 1.f;
          for (int i = 0; i < T; ++i) {
            gm *= sm[lds.alpha + (hc + i) * lds.dks + n];
            sm[lds.qg + i * DK + n] = gm * sm[lds.q + i * DK + n];
            sm[lds.kg + i * DK + n] = gm * sm[lds.k + (hc + i) * lds.dks + n];
          }
        }
      }
    }
    __syncthreads();
  }
  // the next item's checkpoint copy, requested once S is free (same loads on every path). The
  // empty asm marks every S register as read here, on every path: no load into S can still be
  // pending when S is reloaded, so the compiler's waits before the reload stay at zero.
  auto prefetch_next = [&]() {
#pragma unroll
    for (int nt = 0; nt < RT * NT; ++nt) __asm__ volatile("" ::"v"(S[nt]));
#pragma unroll
    for (int tl = 0; tl < RT; ++tl)
      prefetch_ckpt<NT>(a, nit.id, nrt.fold, more && nrt.work, wave * RT + tl, lane, tile(tl));
  };
  const bool lp = reads_lp(prec, fold);

  // ---- matvecs y_i = S q_i (and S k_i for GDN), lane-partial over its columns.
  // A replay item does them right away, which frees S for the next item's
  // checkpoint. A fold item does them on the folded state, further down.
  float yq[RT][TMAX], yk[RT][TMAX];
#pragma unroll
  for (int tl = 0; tl < RT; ++tl) {
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
      yq[tl][i] = 0.f;
      yk[tl][i] = 0.f;
    }
  }
  auto matvec = [&]() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        if (i < T) {
          const float* qi = KDA ? sm + lds.qg + i * DK : sm + lds.q + i * DK;
          const float* ki = KDA ? sm + lds.kg + i * DK : sm + lds.k + (hc + i) * lds.dks;
          const f32x4 qv = ld4(qi + nt * 16 + 4 * g);
          f32x4 kv = f32x4{0.f, 0.f, 0.f, 0.f};
          if (GDN) kv = ld4(ki + nt * 16 + 4 * g);
#pragma unroll
          for (int tl = 0; tl < RT; ++tl) {
            yq[tl][i] = fma4(S[tl * NT + nt], qv, yq[tl][i]);
            if (GDN) yk[tl][i] = fma4(S[tl * NT + nt], kv, yk[tl][i]);
          }
        }
      }
    }
  };

  // The same mat-vecs on the matrix cores, for the delta-rule kinds with 4 or 8 drafts, whose
  // 2 T right-hand vectors q_1..T, k_1..T (KDA: the gated qg, kg) fill half or all of a 16-wide
  // MFMA operand. Y^T = [Q | K]^T S^T is a sum of v_mfma_f32_16x16x4_f32 steps over the
  // checkpoint registers, which are already the B operand: lane (g, col) holds
  // S[row col][16 nt + 4 g + e], i.e. B[k = g][p = col] of step (nt, e), whose four columns are
  // n = 16 nt + 4 k + e. Lane (g, col) supplies A[i = col][k = g], entry 16 nt + 4 g + e of
  // vector i (q_i for i < TMAX, k_{i - TMAX} after; zero for absent drafts and past 2 TMAX),
  // and receives D[4 g + r][col]: vector 4 g + r at its row, summed over every column. Lane
  // group g = i / 4 thus holds vector i's whole sum and the other groups zero, so the group
  // sums of the output phase leave it unchanged.
  auto matvec_mfma = [&]() {
    const int vi = col;
    const bool isq = vi < TMAX;
    const int d = isq ? vi : vi - TMAX;
    const bool live = vi < 2 * TMAX && d < T;
    const float* src = isq ? (KDA ? sm + lds.qg + d * DK : sm + lds.q + d * DK)
                           : (KDA ? sm + lds.kg + d * DK : sm + lds.k + (hc + d) * lds.dks);
    src = (live ? src : sm + lds.q) + 4 * g;
    f32x4 acc[RT];
#pragma unroll
    for (int tl = 0; tl < RT; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 a4 = ld4(src + nt * 16);
      if (!live) a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int tl = 0; tl < RT; ++tl)
          acc[tl] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], S[tl * NT + nt][e], acc[tl], 0, 0, 0);
    }
#pragma unroll
    for (int tl = 0; tl < RT; ++tl) {
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        const int vq = i, vk = TMAX + i;
        yq[tl][i] = (g == (vq >> 2)) ? acc[tl][vq & 3] : 0.f;
        yk[tl][i] = (g == (vk >> 2)) ? acc[tl][vk & 3] : 0.f;
      }
    }
  };

  // ---- 2. decay products and record dot products -----------------------------
  // gq[r + 1][i] = prod of alpha over records (r, hc + i]: the decay of record r
  // at draft i; gk[r + 1][i] the same over (r, hc + i - 1]: at the state just
  // before draft i. Row r0 (r = r0 - 1) holds the checkpoint's factors Gamma_i
  // and Gamma_{i-1}. Entries of records after the end point are zero.
  // Each product set is one suffix-product scan across a wavefront (lane l
  // stands for record first + l), one wavefront per end point.
  auto scans_and_dots = [&]() {
  if (!KDA && outputs) {
    const bool wide = R - r0 + 1 > kWave;
    if (!wide) {
      // (Mamba-2 outputs read only gq: its drafts need no state before them)
      constexpr int kJobsPerDraft = GDN ? 2 : 1;
      for (int job = wave; job < kJobsPerDraft * T; job += W) {
        const int i = GDN ? job >> 1 : job;
        const bool kjob = GDN && (job & 1);
        const int first = r0 - 1, last = R - 1;
        const int e = kjob ? hc + i - 1 : hc + i;
        float* out = sm + (kjob ? lds.gk : lds.gq) + i;
        const int r = first + lane;
        const float x = suffix_product64((r + 1 <= e) ? sm[lds.alpha + r + 1] : 1.f, lane);
        if (r <= last) out[(r + 1) * TMAX] = (r <= e) ? x : 0.f;
      }
    } else {
      for (int t = tid; t < R - r0 + 1; t += nthr) {
        const int r = r0 - 1 + t;
        float* gq = sm + lds.gq + (r + 1) * TMAX;
        float* gk = sm + lds.gk + (r + 1) * TMAX;
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
  }
  if (outputs) {
    // one draft at a time, q_i (and k_i) re-read from LDS per pass: a register
    // copy of every draft's vectors would cost 4 (GDN: 8) registers per draft
    const int sub = lane / LPR, li = lane % LPR;
    if constexpr (CPL == 1) {
      for (int base = r0 + wave * RPI; base < R; base += W * RPI) {
        const int r = base + sub;
        const bool valid = r < R;
        f32x4 kr = f32x4{0.f, 0.f, 0.f, 0.f};
        if (valid) kr = ld4(sm + lds.k + r * lds.dks + 4 * li);
        f32x4 dec = {1.f, 1.f, 1.f, 1.f};  // KDA: gates of records (r, hc + i] for a draft row r
#pragma unroll
        for (int i = 0; i < TMAX; ++i) {
          if (i < T) {
            f32x4 kx = kr;
            const float* qrow = sm + lds.q + i * DK + 4 * li;
            const float* krow = sm + lds.k + (hc + i) * lds.dks + 4 * li;
            if constexpr (KDA) {
              if (r < hc) {
                // a committed row (already carried to the last committed record)
                // meets the drafts' gated vectors
                qrow = sm + lds.qg + i * DK + 4 * li;
                krow = sm + lds.kg + i * DK + 4 * li;
              } else {
                if (i > r - hc) dec *= ld4(sm + lds.alpha + (hc + i) * lds.dks + 4 * li);
                kx = kr * dec;
              }
            }
            const float dq = sum_width<LPR>(dot4(kx, ld4(qrow)));
            if (valid && li == 0) sm[lds.cq + r * TMAX + i] = dq;
            if constexpr (GDN) {
              const float dkk = sum_width<LPR>(dot4(kx, ld4(krow)));
              if (valid && li == 0) sm[lds.ck + r * TMAX + i] = dkk;
            }
          }
        }
      }
    } else {
      // two chunks per lane (Mamba-2 and GDN): chunks li and li + LPR of the row
      for (int base = r0 + wave * RPI; base < R; base += W * RPI) {
        const int r = base + sub;
        const bool valid = r < R;
        const int o0 = 4 * li, o1 = 4 * (li + LPR);
        f32x4 k0 = f32x4{0.f, 0.f, 0.f, 0.f}, k1 = k0;
        if (valid) {
          k0 = ld4(sm + lds.k + r * lds.dks + o0);
          k1 = ld4(sm + lds.k + r * lds.dks + o1);
        }
#pragma unroll
        for (int i = 0; i < TMAX; ++i) {
          if (i < T) {
            const float* qrow = sm + lds.q + i * DK;
            const float dq = sum_width<LPR>(fma4(k1, ld4(qrow + o1), dot4(k0, ld4(qrow + o0))));
            if (valid && li == 0) sm[lds.cq + r * TMAX + i] = dq;
            if constexpr (GDN) {
              const float* krow = sm + lds.k + (hc + i) * lds.dks;
              const float dkk = sum_width<LPR>(fma4(k1, ld4(krow + o1), dot4(k0, ld4(krow + o0))));
              if (valid && li == 0) sm[lds.ck + r * TMAX + i] = dkk;
            }
          }
        }
      }
    }
  }
  };

  // ---- 3. fold: S <- Gamma_h S + sum_j gamma_j v_j k_j^T on MFMA ------------
  // The weights gf_t = prod of alpha over committed records [t, hc) (gf_0 =
  // Gamma_h scales the checkpoint, gf_{j+1} weighs record j) are one
  // suffix-product scan per wavefront: lane t holds gf_t, and gf_hc = 1.
  // GDN with the two-precision checkpoint: the u stored with each committed
  // record was computed from the bf16 copy ("How it works": Gated DeltaNet and
  // Two precisions). Such a fold instead recomputes every correction from the
  // fp32 checkpoint it follows (the staged v rows hold the raw v here), so the
  // bf16 rounding never reaches S. Records go in blocks of 16. With S the state
  // before the block, D_j the decay from the block start to just before record j
  // and g_ij = prod of alpha over (i, j),
  //   w_j = D_j S k_j + sum_{i<j in block} g_ij (k_i . k_j) u_i,  u_j = beta_j (v_j - alpha_j w_j),
  // then S <- D S + sum_i g_i u_i k_i^T over the block (D and g_i to its end). The block's
  // mat-vecs S k_j are one MFMA pass (the 16 keys fill the right-hand operand, as in
  // matvec_mfma), the corrections are solved row by row (a lane per state row, records in
  // order), and the update is one MFMA rank-16 step per tile.
  constexpr int kEB = 8;  // records per block (a divisor of 16: blocks never straddle a Gram block)
  auto exact_fold_state = [&]() {
    // Coefficients c_im = g_im (k_i . k_m) of the records' mutual terms, i < m in one block of
    // 16 (the diagonal blocks of the Gram matrix, scaled by the decays between the two
    // records), by every wavefront (identical values): lane l supplies
    // A[l & 15][l >> 4] = k_{16 jb + (l & 15)}[n] and B[l >> 4][l & 15] = k_{16 jb + (l & 15)}[n]
    // for n = 16 c + 4 (l >> 4) + e; the result gives lane l the product of keys
    // i = l & 15 and m = 4 (l >> 4) + r of block jb, r = 0..3, stored at (i, m).
    for (int jb = 0; 16 * jb < hc; ++jb) {
      const int ja = 16 * jb + col;
      const float* krow = sm + lds.k + (ja < hc ? ja : 0) * lds.dks + 4 * g;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const f32x4 f = ja < hc ? ld4(krow + 16 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f[e], f[e], acc, 0, 0, 0);
      }
      // g_im = prod of alpha over (i, m), walked up from i = col; zero unless i < m
      float gv[4] = {0.f, 0.f, 0.f, 0.f};
      float prod = 1.f;
      for (int m = 0; m < 16; ++m) {
        const float am = sm[lds.alpha + 16 * jb + m];
        if (m > col) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (m == 4 * g + r) gv[r] = prod;
          prod *= am;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sm[lds.gram + jb * 256 + col * 16 + 4 * g + r] = gv[r] * acc[r];
    }
    __builtin_amdgcn_wave_barrier();
    for (int j0 = 0; j0 < hc; j0 += kEB) {
      const int nb = hc - j0 < kEB ? hc - j0 : kEB;
      const float* gblk = sm + lds.gram + (j0 >> 4) * 256 + (j0 & 15) * 17;
      // S k_j for the block's records, every row of the wavefront's tiles: lane (g, col)
      // supplies entry 16 nt + 4 g + e of key j0 + col and receives keys 4 g + r at row col
      {
        const bool live = col < nb;  // (keys past the block: zero)
        const float* src = sm + lds.k + (live ? j0 + col : 0) * lds.dks + 4 * g;
        f32x4 acc[RT];
#pragma unroll
        for (int tl = 0; tl < RT; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 a4 = ld4(src + nt * 16);
          if (!live) a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int tl = 0; tl < RT; ++tl)
              acc[tl] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], S[tl * NT + nt][e], acc[tl], 0, 0, 0);
        }
#pragma unroll
        for (int tl = 0; tl < RT; ++tl)
#pragma unroll
          for (int r = 0; r < 4; ++r) sm[lds.ytab + (4 * g + r) * lds.ys + prow + 16 * tl] = acc[tl][r];
      }
      __builtin_amdgcn_wave_barrier();
      // the corrections, a lane per state row of the wavefront (its RT tiles' 16 RT rows), the
      // records in order; u_j replaces the staged raw v_j (no longer needed)
      if (lane < 16 * RT) {
        const int row = wave * RT * 16 + lane;
        float wp[kEB];
#pragma unroll
        for (int m = 0; m < kEB; ++m) wp[m] = 0.f;
        float Dm = 1.f;
#pragma unroll
        for (int m = 0; m < kEB; ++m) {
          if (m < nb) {
            const int j = j0 + m;
            const float al = sm[lds.alpha + j];
            const float w = Dm * sm[lds.ytab + m * lds.ys + row] + wp[m];
            const float u = sm[lds.beta + j] * (sm[lds.v + j * lds.dvs + row] - al * w);
            sm[lds.v + j * lds.dvs + row] = u;
            // its term in the corrections of the block's later records: row m of the coefficients
#pragma unroll
            for (int m2 = m + 1; m2 < kEB; ++m2) wp[m2] = __builtin_fmaf(gblk[m * 16 + m2], u, wp[m2]);
            Dm *= al;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      // S <- D S + sum_m gamma_m u_m k_m^T: lane t of the scan holds the block's alpha_{j0 + t}
      const float sp = suffix_product64(lane < nb ? sm[lds.alpha + j0 + lane] : 1.f, lane);
      const float D = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sp), 0));
#pragma unroll
      for (int nt = 0; nt < RT * NT; ++nt) S[nt] *= D;
      for (int kc = 0; 4 * kc < nb; ++kc) {
        const int m = 4 * kc + g;
        const bool vj = m < nb;
        const float wm = __shfl(sp, m + 1, kWave);  // prod of alpha over (m, nb): lanes past nb hold 1
        float bval[RT];
#pragma unroll
        for (int tl = 0; tl < RT; ++tl)
          bval[tl] = vj ? wm * sm[lds.v + (j0 + m) * lds.dvs + prow + 16 * tl] : 0.f;
        const float* krow = sm + lds.k + (vj ? j0 + m : 0) * lds.dks + col;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float aval = vj ? krow[nt * 16] : 0.f;
#pragma unroll
          for (int tl = 0; tl < RT; ++tl)
            S[tl * NT + nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bval[tl], S[tl * NT + nt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  };

  auto fold_state = [&]() {
    if constexpr (KIND == kKindGdnExact) {
      exact_fold_state();
#pragma unroll
      for (int tl = 0; tl < RT; ++tl) {
        if (prec != REPLAYSSM_BF16_SHARED) store_hp<NT>(a.hp + hoff, wave * RT + tl, lane, tile(tl));
        if constexpr (NT >= 2) {
          if (prec != REPLAYSSM_FP32)
            store_lp<NT>(a.lp + hoff, wave * RT + tl, lane, tile(tl), prec == REPLAYSSM_BF16_SHARED);
        }
      }
      return;
    }
    // (KDA: the column decay is already applied and the keys carry the rest)
    float gf = 1.f;
    if constexpr (!KDA) {
      gf = suffix_product64((lane < hc) ? sm[lds.alpha + lane] : 1.f, lane);
      const float G = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gf), 0));
#pragma unroll
      for (int nt = 0; nt < RT * NT; ++nt) S[nt] *= G;
    }
    // MFMA 16x16x4 per tile tl: A[m][kk] = k_j[16 nt + m], B[kk][n] = gamma_j v_j[prow - col + 16 tl + n],
    // j = 4 kc + kk; lane l supplies A[l & 15][l >> 4] and B[l >> 4][l & 15].
    const int nkc = (hc + 3) >> 2;
    for (int kc = 0; kc < nkc; ++kc) {
      const int j = 4 * kc + g;
      const bool vj = j < hc;
      const float wj = KDA ? 1.f : __shfl(gf, (j + 1) & (kWave - 1), kWave);  // gf_{j+1}; j + 1 = 64 only if hc = 64
      float bval[RT];
#pragma unroll
      for (int tl = 0; tl < RT; ++tl)
        bval[tl] = vj ? (j + 1 < kWave ? wj : 1.f) * sm[lds.v + j * lds.dvs + prow + 16 * tl] : 0.f;
      const float* krow = sm + lds.k + (vj ? j : 0) * lds.dks + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float aval = vj ? krow[nt * 16] : 0.f;
#pragma unroll
        for (int tl = 0; tl < RT; ++tl)
          S[tl * NT + nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bval[tl], S[tl * NT + nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int tl = 0; tl < RT; ++tl) {
      if (prec != REPLAYSSM_BF16_SHARED) store_hp<NT>(a.hp + hoff, wave * RT + tl, lane, tile(tl));
      if constexpr (NT >= 2) {
        if (prec != REPLAYSSM_FP32)
          store_lp<NT>(a.lp + hoff, wave * RT + tl, lane, tile(tl), prec == REPLAYSSM_BF16_SHARED);
      }
    }
  };

  // ---- 4/5. outputs of the drafts ---------------------------------------------
  // Record r's factors for all drafts are one LDS row of TMAX floats (cq / ck row
  // r, gq / gk row r + 1), read as whole rows so that a record costs one round
  // trip for every draft. After the group sums every lane group holds every
  // draft's value of its rows, so group g stores drafts g, g + 4: a wave writes
  // its drafts with one store instead of one per draft.
  auto row = [&](const float* p, float (&x)[TMAX]) {
    if constexpr (TMAX == 1) {
      x[0] = p[0];
    } else {
#pragma unroll
      for (int c = 0; c < TMAX; c += 4) {
        const f32x4 v = ld4(p + c);
        x[c] = v[0];
        x[c + 1] = v[1];
        x[c + 2] = v[2];
        x[c + 3] = v[3];
      }
    }
  };
  // Lane group g's draft i0 + g, by selects on registers. Each candidate is
  // laundered first: left as plain array reads, the select chain is folded into
  // a lane-dependent index, which sends the array to scratch memory, and the
  // scratch load's wait then drains every outstanding load, the next item's
  // checkpoint prefetch included.
  auto pick = [&](const float (&x)[TMAX], int i0) {
    float r = x[i0];
#pragma unroll
    for (int c = 1; c < 4; ++c) {
      if (i0 + c < TMAX) {
        float xc = x[i0 + c];
        __asm__ volatile("" : "+v"(xc));
        r = (g == c) ? xc : r;
      }
    }
    return r;
  };
  auto write_outputs = [&]() {
  if (outputs) {
    const float* gq = sm + lds.gq;
    const float* gk = sm + lds.gk;
    const float* cq = sm + lds.cq;
    const float* ck = sm + lds.ck;
    const float* sv = sm + lds.v + prow;  // tile tl's value at sv[16 tl]
    float* obase = a.out + ((int64_t)b * T * H + hd) * dv + prow;  // draft 0; draft i is i H dv further
    const int64_t ostep = (int64_t)H * dv;
    float oc[RT][TMAX];
    if constexpr (!GDN) {
      // every staged record r0 .. R - 1 in one pass; the decay rows are zero for
      // records after a draft's end point
      float q0[TMAX];
      row(gq + r0 * TMAX, q0);
#pragma unroll
      for (int tl = 0; tl < RT; ++tl)
#pragma unroll
        for (int i = 0; i < TMAX; ++i) oc[tl][i] = q0[i] * yq[tl][i];
      for (int r = r0 + g; r < R; r += 4) {
        float w[TMAX], c[TMAX];
        row(gq + (r + 1) * TMAX, w);
        row(cq + r * TMAX, c);
#pragma unroll
        for (int tl = 0; tl < RT; ++tl) {
          const float u = sv[r * lds.dvs + 16 * tl];
#pragma unroll
          for (int i = 0; i < TMAX; ++i) oc[tl][i] += w[i] * c[i] * u;
        }
      }
#pragma unroll
      for (int tl = 0; tl < RT; ++tl)
#pragma unroll
        for (int i = 0; i < TMAX; ++i)
          if (i < T) oc[tl][i] = sum_groups(oc[tl][i]);
    } else {
      // committed records in parallel over the four lane groups (KDA: every
      // decay factor is 1, the gates being on the staged vectors)
      float wc[RT][TMAX];
      if constexpr (KDA) {
#pragma unroll
        for (int tl = 0; tl < RT; ++tl) {
#pragma unroll
          for (int i = 0; i < TMAX; ++i) {
            wc[tl][i] = yk[tl][i];
            oc[tl][i] = yq[tl][i];
          }
        }
      } else {
        float k0[TMAX], q0[TMAX];
        row(gk + r0 * TMAX, k0);
        row(gq + r0 * TMAX, q0);
#pragma unroll
        for (int tl = 0; tl < RT; ++tl) {
#pragma unroll
          for (int i = 0; i < TMAX; ++i) {
            wc[tl][i] = k0[i] * yk[tl][i];
            oc[tl][i] = q0[i] * yq[tl][i];
          }
        }
      }
      for (int r = r0 + g; r < hc; r += 4) {
        float kc[TMAX], qc[TMAX];
        row(ck + r * TMAX, kc);
        row(cq + r * TMAX, qc);
        if constexpr (!KDA) {
          float kw[TMAX], qw[TMAX];
          row(gk + (r + 1) * TMAX, kw);
          row(gq + (r + 1) * TMAX, qw);
#pragma unroll
          for (int i = 0; i < TMAX; ++i) {
            kc[i] *= kw[i];
            qc[i] *= qw[i];
          }
        }
#pragma unroll
        for (int tl = 0; tl < RT; ++tl) {
          const float u = sv[r * lds.dvs + 16 * tl];
#pragma unroll
          for (int i = 0; i < TMAX; ++i) {
            wc[tl][i] += kc[i] * u;
            oc[tl][i] += qc[i] * u;
          }
        }
      }
#pragma unroll
      for (int tl = 0; tl < RT; ++tl) {
#pragma unroll
        for (int i = 0; i < TMAX; ++i) {
          if (i < T) {
            wc[tl][i] = sum_groups(wc[tl][i]);
            oc[tl][i] = sum_groups(oc[tl][i]);
          }
        }
      }
      // drafts in order: u_d needs the corrections of the drafts before it; once
      // u_d is known it enters the sums of the drafts after it
      float ud[RT][TMAX];
#pragma unroll
      for (int d = 0; d < TMAX; ++d) {
#pragma unroll
        for (int tl = 0; tl < RT; ++tl) ud[tl][d] = 0.f;
        if (d < T) {
          const float al = KDA ? 1.f : sm[lds.alpha + hc + d];
          const float be = sm[lds.beta + hc + d];
#pragma unroll
          for (int tl = 0; tl < RT; ++tl)
            ud[tl][d] = be * (sv[(hc + d) * lds.dvs + 16 * tl] - al * wc[tl][d]);
          float kc[TMAX], qc[TMAX];
          row(ck + (hc + d) * TMAX, kc);
          row(cq + (hc + d) * TMAX, qc);
          if constexpr (!KDA) {
            float kw[TMAX], qw[TMAX];
            row(gk + (hc + d + 1) * TMAX, kw);
            row(gq + (hc + d + 1) * TMAX, qw);
#pragma unroll
            for (int j = d; j < TMAX; ++j) {
              kc[j] *= kw[j];
              qc[j] *= qw[j];
            }
          }
#pragma unroll
          for (int tl = 0; tl < RT; ++tl) {
#pragma unroll
            for (int j = d; j < TMAX; ++j) {
              if (j > d) wc[tl][j] += kc[j] * ud[tl][d];
              oc[tl][j] += qc[j] * ud[tl][d];
            }
          }
        }
      }
      // the drafts' corrections replace their v in the ring
#pragma unroll
      for (int i0 = 0; i0 < TMAX; i0 += 4) {
        const int i = i0 + g;
        if (i < T) {
          int slot = head + hc + i;
          if (slot >= C) slot -= C;
#pragma unroll
          for (int tl = 0; tl < RT; ++tl) a.ring_v[(bh * C + slot) * dv + prow + 16 * tl] = pick(ud[tl], i0);
        }
      }
    }
#pragma unroll
    for (int i0 = 0; i0 < TMAX; i0 += 4) {
      const int i = i0 + g;
      if (i < T) {
#pragma unroll
        for (int tl = 0; tl < RT; ++tl)
          __builtin_nontemporal_store(pick(oc[tl], i0), obase + i * ostep + 16 * tl);
      }
    }
  }
  };

  // The fold (from the records already in LDS), the mat-vecs on the state the
  // drafts start from, and the next item's checkpoint request, at one program
  // point on every route: the compiler's waits are computed over every
  // control-flow path, and a path without the request would make them drain.
  if constexpr (NT >= 2) {
    if (lp) {  // (the shared-bf16 mode also folds from the bf16 values)
#pragma unroll
      for (int tl = 0; tl < RT; ++tl) widen_lp<NT>(tile(tl));
    }
  }
  if constexpr (KDA) {
    // S Diag(pf): the checkpoint carried over the committed records' gates
    if (work && hc > 0) {
#pragma unroll
      for (int tl = 0; tl < RT; ++tl)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) S[tl * NT + nt] *= ld4(sm + lds.pf + nt * 16 + 4 * g);
    }
  }
  if (fold) fold_state();
  if constexpr (kMfmaMatvec<KIND, TMAX>) {
    if (outputs) matvec_mfma();
  } else {
    if (outputs) matvec();
  }
  prefetch_next();
  scans_and_dots();
  __syncthreads();
  write_outputs();

  // The item's last LDS reads are done once every wavefront is here.
  __syncthreads();
}

// Persistent workgroups: each one walks the (sequence, head) items with a
// stride of the grid size, so that the machine is filled once with as many
// workgroups as fit and none pays a launch per head; consecutive items of the
// grid are neighbours in memory, so the stream over the checkpoints stays
// sequential.
// Advances every sequence's pointers once all items of the launch are done,
// with the same route rule each item applied to the same (old) values: a fold
// moves head past the folded records and adds them to `folded`; decode then
// commits its token (h += 1, p = 0); a fused verify leaves its T drafts
// pending (p = T). Sequences whose items were skipped set their error bit and
// keep their pointers. Run by the last workgroup of the grid to finish (see
// replay_kernel), all its threads striding over the sequences.
__device__ __forceinline__ void commit_pointers(const ReplayArgs& a, int tid, int nthr) {
  for (int b = tid; b < a.B; b += nthr) {
    if (a.select && a.select[b] == 0) continue;
    const SeqPtr p{a.head[b], a.h[b], a.p[b]};
    const Route rt = route_of(a, p);
    if (rt.bad) {
      atomicOr(a.err, rt.corrupt ? REPLAYSSM_DEVERR_CORRUPT : REPLAYSSM_DEVERR_PENDING);
      continue;
    }
    int head = p.head, h = p.h;
    if (rt.fold) {
      head += h;
      if (head >= a.C) head -= a.C;
      a.folded[b] += h;
      h = 0;
    }
    if (a.mode == kModeDecode) {
      h += 1;
      a.p[b] = 0;
    } else if (a.mode == kModeVerify && a.fused) {
      a.p[b] = rt.T;
    }
    a.head[b] = head;
    a.h[b] = h;
  }
}

// (dv <= 256: a workgroup is at most 1024 / RT threads, which also bounds the
// registers the compiler may give a thread)
// Wave priority by progress. A compute unit issues from its oldest waves first, so of the
// workgroups sharing it the ones dispatched first get through their equal shares of items
// sooner (measured: a Mamba-2 decode launch's first-dispatched workgroups end about 20 % before
// the last-dispatched ones), and the launch waits for the slowest. Each workgroup lowers its
// waves' priority by one step per quarter of its share: one that is ahead yields the issue slots
// to those behind it. Measured at B = 256 against no priority change: GDN and KDA decode -3 to
// -4 %, verify T = 4 -1.6 to -3 % (all kinds); Mamba-2 decode unchanged with the fp32
// checkpoint and 1.4 % slower with the bf16 copy, so its one-draft kernels keep one priority.
template <int KIND, int TMAX>
constexpr bool kLevelled = !(KIND == REPLAYSSM_MAMBA2 && TMAX == 1);

__device__ __forceinline__ void level_priority(int done, int share) {
  int lvl = 3 - (4 * done) / share;
  lvl = __builtin_amdgcn_readfirstlane(lvl < 0 ? 0 : lvl);
  // (the priority is an immediate operand)
  if (lvl == 3) __builtin_amdgcn_s_setprio(3);
  else if (lvl == 2) __builtin_amdgcn_s_setprio(2);
  else if (lvl == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

template <int KIND, int NT, int TMAX, bool FUSED, int RT>
__global__ void __launch_bounds__(1024 / RT) replay_kernel(const ReplayArgs a) {
  extern __shared__ f32x4 smem_v4[];
  float* sm = reinterpret_cast<float*>(smem_v4);
  const int items = a.B * a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = gridDim.x;
  // Pointers of the workgroup's items are read 64 at a time, one item per
  // lane, and handed to each item with readlane: no memory round trip per item.
  int ph = 0, phc = 0, pp = 0;
  auto batch = [&](int first_item) {
    const int it = first_item + lane * G;
    if (it < items) {
      const int bb = it / a.H;
      ph = a.head[bb];
      phc = a.h[bb];
      pp = a.p[bb];
      if (a.select && a.select[bb] == 0) phc = 0;  // a selective flush leaves it alone
    }
    // Wait for them here, once per batch. Left pending, they would be the
    // newest loads on one path into the next item and the oldest on the other,
    // and the wait at their first use would have to drain every load.
    __asm__ volatile("" ::"v"(ph), "v"(phc), "v"(pp));
  };
  auto ptr_at = [&](int kl) {
    return SeqPtr{__builtin_amdgcn_readlane(ph, kl), __builtin_amdgcn_readlane(phc, kl),
                  __builtin_amdgcn_readlane(pp, kl)};
  };
  batch(blockIdx.x);  // (a workgroup without items still arrives at the end)
  SeqPtr ptr = ptr_at(0);
  Route rt = route_of(a, ptr);
  const bool any = (int)blockIdx.x < items;
  if (!any) rt.work = false;
  f32x4 S[RT * NT];
  RecRegs<TMAX, RT> rr;
  // Loop invariants of the workgroup: the LDS carve-up and where a thread's
  // share of the ring rows lies.
  const ReplayLds lds(a.C, NT * 16, a.dv, TMAX, KIND, a.lds_unpadded != 0);
  const StageMap map(threadIdx.x, blockDim.x, NT * 4, a.dv);
  // Items advance by the grid size G: (sequence, head) advances by (G / H, G % H)
  // with a carry, so no item divides by H.
  const int H = a.H;
  const int step_b = G / H, step_h = G - step_b * H;
  auto advance = [&](const Item& x) {
    Item n{x.id + G, x.b + step_b, x.hd + step_h};
    if (n.hd >= H) {
      n.hd -= H;
      ++n.b;
    }
    return n;
  };
  Item it{(int)blockIdx.x, (int)blockIdx.x / H, (int)blockIdx.x % H};
  load_records<KIND, NT, TMAX, FUSED, RT>(a, it, ptr, rt, any, threadIdx.x, map, rr);
  {
    using Tile = f32x4[NT];
#pragma unroll
    for (int tl = 0; tl < RT; ++tl)
      prefetch_ckpt<NT>(a, it.id, rt.fold, any && rt.work, wave * RT + tl, lane,
                        *reinterpret_cast<Tile*>(&S[tl * NT]));
  }
  for (int k = 0; it.id < items; ++k) {
    if constexpr (kLevelled<KIND, TMAX>) level_priority(k, (items + G - 1) / G);
    const Item nit = advance(it);
    const int kn = (k + 1) & 63;
    if (kn == 0 && nit.id < items) batch(nit.id);
    const SeqPtr nptr = ptr_at(kn);
    const Route nrt = route_of(a, nptr);
    replay_item<KIND, NT, TMAX, FUSED, RT>(a, sm, lds, map, it, ptr, rt, S, rr, nit, nptr, nrt);
    it = nit;
    ptr = nptr;
    rt = nrt;
  }

  // Pointer commit. Each workgroup arrives once, after its last item (all its
  // pointer reads are behind it); the last one to arrive applies the rule to
  // every sequence. Nothing is published through the counter, so no fence is
  // needed (see arrive_last); the new pointers reach the next kernel at the
  // kernel boundary. One relaxed atomic per workgroup and launch, at its end.
  int* flag = reinterpret_cast<int*>(sm);
  if (threadIdx.x == 0) flag[0] = arrive_last(a.arrive, 0, G) ? 1 : 0;
  __syncthreads();
  if (flag[0]) commit_pointers(a, threadIdx.x, blockDim.x);
}

// How one instantiation runs a call: its dynamic LDS (record rows padded or not) and the
// workgroups of it that fit on a compute unit. Padded rows (no bank conflicts) unless unpadded
// ones let more workgroups share a compute unit where the padded carve leaves fewer than four
// (long windows, whose staging then sets the occupancy). Measured at B=256, Mamba-2 64x128:
// L=64, T=1 two -> three workgroups, 3.72 -> 4.76 TB/s; L=32, T=8 three -> four, +8 %; but
// L=32, T=4 four -> five ran 20 % slower (the bank conflicts of unpadded rows cost more than
// the fifth workgroup).
struct LaunchPlan {
  int unpadded;
  size_t smem;
  int per_cu;
};

// Raises the dynamic LDS a launch of `fn` may request (beyond 64 KiB), once per device and size.
static hipError_t allow_lds(const void* fn, size_t smem) {
  if (smem <= 64 * 1024) return hipSuccess;
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> raised[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& x : raised[dev])
    if (x.first == fn && x.second >= (int)smem) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  raised[dev].push_back({fn, (int)smem});
  return hipSuccess;
}

template <int KIND, int NT, int TMAX, bool FUSED, int RT>
static hipError_t plan_t(const ReplayArgs& a, LaunchPlan* plan) {
  const int block = a.dv / (16 * RT) * kWave;
  const void* fn = reinterpret_cast<const void*>(&replay_kernel<KIND, NT, TMAX, FUSED, RT>);
  const ReplayLds padded(a.C, NT * 16, a.dv, TMAX, KIND, false), unpadded(a.C, NT * 16, a.dv, TMAX, KIND, true);
  hipError_t e = allow_lds(fn, (size_t)padded.total * 4);
  if (e != hipSuccess) return e;
  int occ_p = 0;
  e = blocks_per_cu(fn, block, (size_t)padded.total * 4, &occ_p);
  if (e != hipSuccess) return e;
  *plan = LaunchPlan{0, (size_t)padded.total * 4, occ_p};
  if (unpadded.total < padded.total && occ_p < 4) {
    int occ_u = 0;
    e = blocks_per_cu(fn, block, (size_t)unpadded.total * 4, &occ_u);
    if (e != hipSuccess) return e;
    if (occ_u > occ_p) *plan = LaunchPlan{1, (size_t)unpadded.total * 4, occ_u};
  }
  return hipSuccess;
}

template <int KIND, int NT, int TMAX, bool FUSED, int RT>
static hipError_t launch_t(const ReplayArgs& args, hipStream_t s) {
  const int block = args.dv / (16 * RT) * kWave;
  const void* fn = reinterpret_cast<const void*>(&replay_kernel<KIND, NT, TMAX, FUSED, RT>);
  LaunchPlan plan;
  hipError_t e = plan_t<KIND, NT, TMAX, FUSED, RT>(args, &plan);
  if (e != hipSuccess) return e;
  ReplayArgs a = args;
  a.lds_unpadded = plan.unpadded;
  int grid = 0;
  e = persistent_grid(fn, block, plan.smem, a.B * a.H, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((replay_kernel<KIND, NT, TMAX, FUSED, RT>), dim3((unsigned)grid), dim3((unsigned)block),
                     plan.smem, s, a);
  return hipGetLastError();
}

// dk = 128 with at most four drafts: two 16-row tiles per wavefront, so that the
// per-record factor rows read from LDS, the staged q / k chunks of the mat-vecs,
// the scans, the dot passes and (exact-correction fold) the Gram blocks serve 32
// state rows instead of 16, at twice the state registers. Each row's arithmetic is the same in both forms (same lanes,
// same order), so the results are bit-identical.
template <int KIND, int NT, int TMAX>
constexpr bool kTwoTiles = NT == 8 && TMAX <= 4;

std::atomic<int> g_tiling{REPLAYSSM_TILES_AUTO};

void set_tiling(int policy) { g_tiling.store(policy, std::memory_order_relaxed); }
int get_tiling() { return g_tiling.load(std::memory_order_relaxed); }

// Automatic choice: two tiles once the batch fills the device (their occupancy
// holds more heads in flight per compute unit), one below that (a head's work
// spread over twice the wavefronts finishes sooner). Thresholds from B-sweeps of
// decode and verify T = 4 on MI355X: Mamba-2 64x128 (dv = 64) breaks even at 64
// items per CU, Gated DeltaNet and KDA 128x128 (dv = 128) at about 6, and the
// exact-correction fold of Gated DeltaNet's two-precision checkpoint, whose fold
// work the second tile shares, at about 3.
static hipError_t two_tiles(const ReplayArgs& a, bool exact, bool* two) {
  *two = false;
  if (a.dv % 32 != 0) return hipSuccess;
  const int policy = get_tiling();
  if (policy != REPLAYSSM_TILES_AUTO) {
    *two = policy == REPLAYSSM_TILES_TWO;
    return hipSuccess;
  }
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int64_t per_cu = a.dv < 128 ? 64 : exact ? 3 : 6;
  *two = (int64_t)a.B * a.H >= per_cu * cus;
  return hipSuccess;
}

template <int KIND, int NT, int TMAX, int RT>
static hipError_t launch_r(const ReplayArgs& a, hipStream_t s) {
  return a.fused ? launch_t<KIND, NT, TMAX, true, RT>(a, s) : launch_t<KIND, NT, TMAX, false, RT>(a, s);
}

// Two tiles also need to put more items in flight than one: where the record staging's LDS
// holds both forms to the same workgroups per compute unit (long windows), one tile's twice as
// many wavefronts finish each item sooner. Measured at B=256, Mamba-2 64x128, one against two
// tiles: L=64, T=1 0.71 against 0.61 M tokens/s; L=64, T=4 0.86 against 0.62 M accepted
// tokens/s; L=32, T=4 1.31 against 1.25 M; L=16 within 0.5 %.
template <int KIND, int NT, int TMAX>
static hipError_t more_in_flight_with_two(const ReplayArgs& a, bool* two) {
  LaunchPlan p1, p2;
  hipError_t e = a.fused ? plan_t<KIND, NT, TMAX, true, 1>(a, &p1) : plan_t<KIND, NT, TMAX, false, 1>(a, &p1);
  if (e != hipSuccess) return e;
  e = a.fused ? plan_t<KIND, NT, TMAX, true, 2>(a, &p2) : plan_t<KIND, NT, TMAX, false, 2>(a, &p2);
  if (e != hipSuccess) return e;
  *two = p2.per_cu > p1.per_cu;
  return hipSuccess;
}

template <int KIND, int NT, int TMAX>
static hipError_t launch_f(const ReplayArgs& a, hipStream_t s) {
  if constexpr (kTwoTiles<KIND, NT, TMAX>) {
    bool two = false;
    hipError_t e = two_tiles(a, KIND == kKindGdnExact, &two);
    if (e != hipSuccess) return e;
    if (two && get_tiling() == REPLAYSSM_TILES_AUTO) {
      e = more_in_flight_with_two<KIND, NT, TMAX>(a, &two);
      if (e != hipSuccess) return e;
    }
    if (two) return launch_r<KIND, NT, TMAX, 2>(a, s);
  }
  return launch_r<KIND, NT, TMAX, 1>(a, s);
}

template <int KIND, int NT>
static hipError_t launch_nt(int tmax, const ReplayArgs& a, hipStream_t s) {
  switch (tmax) {
    case 1: return launch_f<KIND, NT, 1>(a, s);
    case 4: return launch_f<KIND, NT, 4>(a, s);
    case 8: return launch_f<KIND, NT, 8>(a, s);
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
  if (kind == REPLAYSSM_GDN && a.precision == REPLAYSSM_FP32_HP_BF16_LP)
    return launch_kind<kKindGdnExact>(dk, tmax, a, s);
  if (kind == REPLAYSSM_KDA) return launch_kind<REPLAYSSM_KDA>(dk, tmax, a, s);
  return kind == REPLAYSSM_GDN ? launch_kind<REPLAYSSM_GDN>(dk, tmax, a, s)
                               : launch_kind<REPLAYSSM_MAMBA2>(dk, tmax, a, s);
}

}  // namespace rs
