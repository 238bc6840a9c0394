// Per-sequence routing of the replay kernel.
#pragma once

#include "device.hpp"

namespace rs {

// A sequence's buffer pointers as one item reads them.
struct SeqPtr {
  int head, h, p;
};

// What one item does, from its sequence's pointers (the same in every
// workgroup of the sequence).
struct Route {
  int T;        // drafts of this call (0 for flush)
  bool corrupt; // pointers outside their invariant ranges
  bool bad;     // corrupt, or a decode/verify call whose pending count is not T
  bool fold;    // fold the committed records into the checkpoint first
  bool work;    // anything to do for this item
  bool outputs; // produce draft outputs
  int R;        // staged records: committed [0, h), drafts [h, h + T)
  int r0;       // first record replayed on top of the checkpoint
};

__device__ __forceinline__ Route route_of(const ReplayArgs& a, const SeqPtr& p) {
  Route r;
  r.T = (a.mode == kModeFlush) ? 0 : a.T;
  r.corrupt = p.head < 0 || p.head >= a.C || p.h < 0 || p.h > a.L || p.p < 0 || p.p > a.C - a.L;
  // decode/verify consume T pending drafts; the fused calls append them first (p = 0 on entry)
  r.bad = r.corrupt || ((a.mode != kModeFlush) && (p.p != (a.fused ? 0 : r.T)));
  r.fold = !r.bad && ((a.mode == kModeFlush) ? (p.h > 0) : (p.h + r.T > a.L));
  r.work = !r.bad && (a.mode != kModeFlush || r.fold);
  r.outputs = r.work && (a.mode != kModeFlush);
  r.R = p.h + r.T;
  r.r0 = r.fold ? p.h : 0;
  return r;
}

__device__ __forceinline__ int ring_slot(int head, int r, int C) {
  const int s = head + r;
  return s >= C ? s - C : s;
}

}  // namespace rs
