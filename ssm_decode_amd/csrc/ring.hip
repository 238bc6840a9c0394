// Buffer and pointer kernels of libreplayssm: append, accept, init, and the
// conversions between the logical checkpoint order and the private layouts.
#include <mutex>
#include <vector>

#include "device.hpp"

namespace rs {

hipError_t device_cus(int* cus) {
  static std::mutex mu;
  static int count[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (count[dev] == 0) {
    e = hipDeviceGetAttribute(&count[dev], hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  *cus = count[dev];
  return hipSuccess;
}

hipError_t device_max_lds(int* bytes) {
  static std::mutex mu;
  static int lds[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (lds[dev] == 0) {
    int per_block = 0, optin = 0;
    e = hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    // (the opt-in figure, where the runtime reports one, is what a launch may request)
    if (hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) != hipSuccess) optin = 0;
    lds[dev] = optin > per_block ? optin : per_block;
  }
  *bytes = lds[dev];
  return hipSuccess;
}

hipError_t persistent_grid(const void* kernel, int block, size_t smem, int items, int* grid) {
  int per_cu = 0, cus = 0;
  hipError_t e = blocks_per_cu(kernel, block, smem, &per_cu);
  if (e != hipSuccess) return e;
  e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const long g = (long)cus * per_cu;
  *grid = (int)(g < items ? g : items);
  if (*grid < 1) *grid = 1;
  return hipSuccess;
}

hipError_t blocks_per_cu(const void* kernel, int block, size_t smem, int* per_cu_out) {
  struct Entry {
    const void* kernel;
    int block;
    size_t smem;
    int device;
    int per_cu;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int per_cu = -1;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& x : cache)
    if (x.kernel == kernel && x.block == block && x.smem == smem && x.device == dev) per_cu = x.per_cu;
  if (per_cu < 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, smem);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    cache.push_back(Entry{kernel, block, smem, dev, per_cu});
  }
  *per_cu_out = per_cu;
  return hipSuccess;
}

// A record's decay from its raw time step: Delta = softplus(dt + dt_bias[h]),
// alpha = exp(-Delta A[h]), softplus in the form max(x, 0) + log1p(e^-|x|),
// which neither overflows for large x nor loses the small values for x << 0.
__device__ __forceinline__ float decay_from_dt(const AppendArgs& a, int64_t src, int hd) {
  const float x = a.dt[src] + (a.dt_bias ? a.dt_bias[hd] : 0.f);
  const float delta = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
  return expf(-delta * a.A[hd]);
}

// Append: the T new records of every head of sequence b go to ring slots
// (head + h + p + i) mod C ("ReplaySSM: Cache SSM Inputs, Not State", How it
// works: each step appends its inputs; drafts are appended together and the
// buffer is circular with capacity L + T). Grid (chunks, B): the chunks of a
// sequence copy its k and v rows as float4 units; the source side is one
// contiguous span per sequence. The last chunk to finish publishes p += T.
template <int KIND>
__global__ void __launch_bounds__(256) append_kernel(const AppendArgs a) {
  const int b = blockIdx.y;
  const int head = a.head[b], hc = a.h[b], pend = a.p[b];
  const int T = a.T, H = a.H, C = a.C, dk = a.dk, dv = a.dv;
  const int L = C - a.T_max;
  const bool corrupt = head < 0 || head >= C || hc < 0 || hc > L || pend < 0;
  const bool bad = corrupt || pend + T > a.T_max;
  const int first = head + hc + pend;
  if (!bad) {
    const int dk4 = dk >> 2, dv4 = dv >> 2;
    const int nk = T * H * dk4;
    const float* ksrc = a.k + (int64_t)b * T * H * dk;
    const float* vsrc = a.v + (int64_t)b * T * H * dv;
    // units: the k rows, then (KDA) the gate rows, then the v rows
    const int nka = KIND == REPLAYSSM_KDA ? 2 * nk : nk;
    const float* asrc = a.alpha + (int64_t)b * T * H * dk;
    for (int u = blockIdx.x * 256 + threadIdx.x; u < a.units_per_seq; u += gridDim.x * 256) {
      if (u < nka) {
        const bool gate = u >= nk;
        const int uk = gate ? u - nk : u;
        const int c4 = uk % dk4, th = uk / dk4;
        const int hd = th % H, i = th / H;
        const int slot = (first + i) % C;
        const int64_t dst = (((int64_t)b * H + hd) * C + slot) * dk + 4 * c4;
        if (gate)
          st4(a.ring_alpha + dst, ld4(asrc + 4 * (int64_t)uk));
        else
          st4(a.ring_k + dst, ld4(ksrc + 4 * (int64_t)uk));
      } else {
        const int uv = u - nka;
        const int c4 = uv % dv4, th = uv / dv4;
        const int hd = th % H, i = th / H;
        const int slot = (first + i) % C;
        const int64_t dst = (((int64_t)b * H + hd) * C + slot) * dv + 4 * c4;
        const f32x4 x = ld4(vsrc + 4 * (int64_t)uv);
        st4(a.ring_v + dst, x);
        if (KIND != REPLAYSSM_MAMBA2 && a.ring_vraw) st4(a.ring_vraw + dst, x);
      }
    }
    if (blockIdx.x == 0) {
      for (int u = threadIdx.x; u < T * H; u += 256) {
        const int hd = u % H, i = u / H;
        const int slot = (first + i) % C;
        const int64_t dst = ((int64_t)b * H + hd) * C + slot;
        const int64_t src = ((int64_t)b * T + i) * H + hd;
        if (KIND != REPLAYSSM_KDA) a.ring_alpha[dst] = a.dt ? decay_from_dt(a, src, hd) : a.alpha[src];
        if (KIND != REPLAYSSM_MAMBA2) a.ring_beta[dst] = a.beta[src];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && arrive_last(a.arrive, b, gridDim.x)) {
    if (bad)
      atomicOr(a.err, corrupt ? REPLAYSSM_DEVERR_CORRUPT : REPLAYSSM_DEVERR_APPEND_OVERFLOW);
    else
      a.p[b] = pend + T;
  }
}

// ---- replayssm_append_static: the append without the caller's scratch -------------
// The append's per-sequence arrival counters live in this array instead of
// state->arrive, for callers that cannot allocate. Each GPU the library runs on
// holds its own copy (zero at load) until the process ends. In host code the
// name is only a stand-in: the device address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) int32_t scratch[kStaticScratchSeqs];

// Device address of `scratch` on the current device.
static hipError_t static_scratch(int32_t** out) {
  static std::mutex mu;
  static int32_t* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<int32_t*>(ptr);
  }
  *out = addr[dev];
  return hipSuccess;
}

// Zeroes n counters (a kernel, not a memset, so that the call can be captured in
// a graph and replayed).
__global__ void __launch_bounds__(256) clear_counters_kernel(int32_t* c, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) c[i] = 0;
}

hipError_t launch_append(int kind, const AppendArgs& a, hipStream_t s);

hipError_t launch_append_static(int kind, const AppendArgs& args, hipStream_t s) {
  if (args.B > kStaticScratchSeqs) return hipErrorInvalidValue;  // (the entry point rejects it first)
  int32_t* counters = nullptr;
  hipError_t e = static_scratch(&counters);
  if (e != hipSuccess) return e;
  // the array keeps what the last call on this device left there: this call's counters start at zero
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((args.B + 255) / 256)), dim3(256), 0, s, counters,
                     args.B);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  AppendArgs a = args;
  a.arrive = counters;
  return launch_append(kind, a, s);
}

hipError_t launch_append(int kind, const AppendArgs& a, hipStream_t s) {
  const int per_block = 256 * 4;
  int chunks = (a.units_per_seq + per_block - 1) / per_block;
  if (chunks < 1) chunks = 1;
  const dim3 grid((unsigned)chunks, (unsigned)a.B);
  if (kind == REPLAYSSM_KDA)
    hipLaunchKernelGGL(append_kernel<REPLAYSSM_KDA>, grid, dim3(256), 0, s, a);
  else if (kind == REPLAYSSM_GDN)
    hipLaunchKernelGGL(append_kernel<REPLAYSSM_GDN>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<REPLAYSSM_MAMBA2>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Accept: the accepted prefix only moves the pointer (h += a, p = 0); rejected
// records stay where they are until the next append overwrites them ("How it
// works": Speculative decoding).
__global__ void __launch_bounds__(256) accept_kernel(int32_t* h, int32_t* p, int32_t* err,
                                                     const int32_t* acc, int B, int L) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int hb = h[b], pb = p[b];
  if (hb < 0 || hb > L || pb < 0) {
    atomicOr(err, REPLAYSSM_DEVERR_CORRUPT);
    return;
  }
  int lim = L - hb < pb ? L - hb : pb;
  if (lim < 0) lim = 0;
  int ab = acc[b];
  if (ab < 0 || ab > lim) {
    atomicOr(err, REPLAYSSM_DEVERR_ACCEPT);
    ab = ab < 0 ? 0 : lim;
  }
  h[b] = hb + ab;
  p[b] = 0;
}

hipError_t launch_accept(int32_t* h, int32_t* p, int32_t* err, const int32_t* acc, int B, int L,
                         hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, h, p, err,
                     acc, B, L);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) init_kernel(int32_t* head, int32_t* h, int32_t* p,
                                                   int64_t* folded, int32_t* arrive, int32_t* err,
                                                   int B) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b == 0) *err = 0;
  if (b >= B) return;
  head[b] = 0;
  h[b] = 0;
  p[b] = 0;
  folded[b] = 0;
  arrive[b] = 0;
}

hipError_t launch_init(int32_t* head, int32_t* h, int32_t* p, int64_t* folded, int32_t* arrive,
                       int32_t* err, int B, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, head, h, p,
                     folded, arrive, err, B);
  return hipGetLastError();
}

// Logical [heads][dv][dk] fp32 <-> private tile layouts. One thread per
// (head, tile, lane): four consecutive columns of one row.
__global__ void __launch_bounds__(256) pack_kernel(const float* src, float* hp, uint16_t* lp,
                                                   int64_t nheads, int dv, int dk) {
  const int NT = dk >> 4, PT = dv >> 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nheads * PT * NT * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t t = gid >> 6;
  const int tile = (int)(t % (PT * NT));
  const int64_t hh = t / (PT * NT);
  const int pt = tile / NT, nt = tile - pt * NT;
  const int p = 16 * pt + (lane & 15), n = 16 * nt + 4 * (lane >> 4);
  const int64_t base = hh * (int64_t)dv * dk;
  const f32x4 x = ld4(src + base + (int64_t)p * dk + n);
  if (hp) st4(hp + base + tile * 256 + lane * 4, x);
  if (lp) {
    uint2* d = reinterpret_cast<uint2*>(lp + base + (pt * (NT / 2) + nt / 2) * 512 + lane * 8 +
                                        (nt & 1) * 4);
    *d = uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
}

__global__ void __launch_bounds__(256) unpack_kernel(const float* hp, const uint16_t* lp, float* dst,
                                                     int64_t nheads, int dv, int dk) {
  const int NT = dk >> 4, PT = dv >> 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nheads * PT * NT * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t t = gid >> 6;
  const int tile = (int)(t % (PT * NT));
  const int64_t hh = t / (PT * NT);
  const int pt = tile / NT, nt = tile - pt * NT;
  const int p = 16 * pt + (lane & 15), n = 16 * nt + 4 * (lane >> 4);
  const int64_t base = hh * (int64_t)dv * dk;
  f32x4 x;
  if (hp) {
    x = ld4(hp + base + tile * 256 + lane * 4);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(lp + base + (pt * (NT / 2) + nt / 2) * 512 +
                                                     lane * 8 + (nt & 1) * 4);
    x = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
  }
  st4(dst + base + (int64_t)p * dk + n, x);
}

hipError_t launch_pack(const float* src, float* hp, uint16_t* lp, int64_t nheads, int dv, int dk,
                       hipStream_t s) {
  const int64_t threads = nheads * (dv / 16) * (dk / 16) * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, src, hp,
                     lp, nheads, dv, dk);
  return hipGetLastError();
}

// Prefix states. A cached prefix is shared between sequences as a plain state:
// the checkpoint of a sequence whose committed records are all folded (the
// checkpoint alone trails the tokens by the unfolded records, the staleness
// raised in the thread's replies on prefix caching). One thread per (listed
// sequence, head, tile, lane), as in pack/unpack; indices outside 0..B-1 are
// skipped and flagged.
__global__ void __launch_bounds__(256) snapshot_kernel(const float* hp, const uint16_t* lp, const int32_t* h,
                                                       int32_t* err, const int32_t* seqs, int n, float* dst,
                                                       int B, int H, int dv, int dk) {
  const int NT = dk >> 4, PT = dv >> 4;
  const int64_t per_seq = (int64_t)H * PT * NT * 64;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)n * per_seq) return;
  const int i = (int)(gid / per_seq);
  const int b = seqs[i];
  const int64_t rest = gid - (int64_t)i * per_seq;
  if (b < 0 || b >= B) {
    if (rest == 0) atomicOr(err, REPLAYSSM_DEVERR_INDEX);
    return;
  }
  if (rest == 0 && h[b] != 0) atomicOr(err, REPLAYSSM_DEVERR_STALE);
  const int lane = (int)(rest & 63);
  const int64_t t = rest >> 6;
  const int tile = (int)(t % (PT * NT));
  const int hd = (int)(t / (PT * NT));
  const int pt = tile / NT, nt = tile - pt * NT;
  const int pr = 16 * pt + (lane & 15), nc = 16 * nt + 4 * (lane >> 4);
  const int64_t src_base = ((int64_t)b * H + hd) * dv * dk;
  f32x4 x;
  if (hp) {
    x = ld4(hp + src_base + tile * 256 + lane * 4);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(lp + src_base + (pt * (NT / 2) + nt / 2) * 512 + lane * 8 +
                                                     (nt & 1) * 4);
    x = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
  }
  st4(dst + ((int64_t)i * H + hd) * dv * dk + (int64_t)pr * dk + nc, x);
}

__global__ void __launch_bounds__(256) restore_kernel(float* hp, uint16_t* lp, int32_t* head, int32_t* h,
                                                      int32_t* p, int64_t* folded, int32_t* err,
                                                      const int32_t* seqs, int n, const float* src, int B, int H,
                                                      int dv, int dk) {
  const int NT = dk >> 4, PT = dv >> 4;
  const int64_t per_seq = (int64_t)H * PT * NT * 64;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)n * per_seq) return;
  const int i = (int)(gid / per_seq);
  const int b = seqs[i];
  const int64_t rest = gid - (int64_t)i * per_seq;
  if (b < 0 || b >= B) {
    if (rest == 0) atomicOr(err, REPLAYSSM_DEVERR_INDEX);
    return;
  }
  if (rest == 0) {
    head[b] = 0;
    h[b] = 0;
    p[b] = 0;
    folded[b] = 0;
  }
  const int lane = (int)(rest & 63);
  const int64_t t = rest >> 6;
  const int tile = (int)(t % (PT * NT));
  const int hd = (int)(t / (PT * NT));
  const int pt = tile / NT, nt = tile - pt * NT;
  const int pr = 16 * pt + (lane & 15), nc = 16 * nt + 4 * (lane >> 4);
  const f32x4 x = ld4(src + ((int64_t)i * H + hd) * dv * dk + (int64_t)pr * dk + nc);
  const int64_t dst_base = ((int64_t)b * H + hd) * dv * dk;
  if (hp) st4(hp + dst_base + tile * 256 + lane * 4, x);
  if (lp) {
    uint2* d = reinterpret_cast<uint2*>(lp + dst_base + (pt * (NT / 2) + nt / 2) * 512 + lane * 8 + (nt & 1) * 4);
    *d = uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
}

hipError_t launch_snapshot(const float* hp, const uint16_t* lp, const int32_t* h, int32_t* err,
                           const int32_t* seqs, int n, float* dst, int B, int H, int dv, int dk,
                           hipStream_t s) {
  const int64_t threads = (int64_t)n * H * (dv / 16) * (dk / 16) * 64;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(snapshot_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, hp, lp, h, err,
                     seqs, n, dst, B, H, dv, dk);
  return hipGetLastError();
}

hipError_t launch_restore(float* hp, uint16_t* lp, int32_t* head, int32_t* h, int32_t* p, int64_t* folded,
                          int32_t* err, const int32_t* seqs, int n, const float* src, int B, int H, int dv,
                          int dk, hipStream_t s) {
  const int64_t threads = (int64_t)n * H * (dv / 16) * (dk / 16) * 64;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(restore_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, hp, lp, head, h, p,
                     folded, err, seqs, n, src, B, H, dv, dk);
  return hipGetLastError();
}

hipError_t launch_unpack(const float* hp, const uint16_t* lp, float* dst, int64_t nheads, int dv,
                         int dk, hipStream_t s) {
  const int64_t threads = nheads * (dv / 16) * (dk / 16) * 64;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, hp,
                     lp, dst, nheads, dv, dk);
  return hipGetLastError();
}

}  // namespace rs
