// Work order of the prefill kernels (bf16 and fp8 forward): which (head, query tile) a
// workgroup takes.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Workgroups are dealt to the 8 XCDs round-robin (block i runs on XCD i % 8). Each XCD
// gets whole heads, so their K/V stay in that XCD's L2, and walks them heaviest query
// tiles first (largest-first scheduling keeps the causal tail short; rr = 0 is the
// heaviest tile rank). With at least 32 query tiles per head it takes its heads four at a
// time, so the workgroups running together on it stream the K/V of four heads, not of all
// of them, and their L2 serves more of the re-reads with the load balance unchanged (with
// fewer tiles per head the grouping lengthens the causal tail). Shapes that do not split
// evenly over the XCDs use one global heaviest-first order. The map from block to
// (hl, rr) is a bijection onto [0, heads) x [0, n_qt).
__device__ __forceinline__ void prefill_work_unit(int block, int heads, int n_qt, int& hl, int& rr) {
  const int total = heads * n_qt;
  if ((total & 7) == 0 && ((total >> 3) % n_qt) == 0) {
    const int hpx = (total >> 3) / n_qt;                      // heads per XCD
    const int G = (n_qt >= 32 && (hpx & 3) == 0) ? 4 : hpx;   // heads walked together
    const int li = block >> 3;
    const int grp = li / (G * n_qt);
    const int r = li - grp * G * n_qt;
    rr = r / G;
    hl = (block & 7) * hpx + grp * G + (r - rr * G);
  } else {
    rr = block / heads;
    hl = block - rr * heads;
  }
}

}  // namespace fa
