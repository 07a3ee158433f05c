// Device helpers shared by the gfx950 kernels of libuf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define UF_LDS __attribute__((address_space(3)))
#define UF_GLOBAL __attribute__((address_space(1)))

namespace uf {

constexpr int kXcds = 8;        // MI355X: 8 XCDs, work-groups dealt round-robin

// Work-group b is dispatched to XCD b % 8.  Renumber so that each XCD gets
// one contiguous run of work items (neighbouring query blocks of the same
// head), which then share K/V tiles in that XCD's L2.
__device__ inline int xcd_contiguous(int b, int n) {
  const int per = n / kXcds, extra = n % kXcds;
  const int xcd = b % kXcds, slot = b / kXcds;
  return xcd * per + min(xcd, extra) + slot;
}

// Windowed order: work items are taken in windows of kXcds * kRun consecutive items, and
// within a window each XCD gets kRun consecutive ones (kRun = the work-groups an XCD holds at
// once: 32 CUs x 2).  All XCDs then work inside one window at a time, which keeps the
// chip-wide working set (heads in flight) small for the last-level cache, while each XCD's
// resident work-groups still hold neighbouring items for its L2.  The last, partial window
// is split XCD-contiguously.
constexpr int kRun = 64;
__device__ inline int xcd_windowed(int b, int n) {
  constexpr int W = kXcds * kRun;
  const int full = (n / W) * W;
  if (b >= full) return full + xcd_contiguous(b - full, n - full);
  const int xcd = b % kXcds, slot = b / kXcds;
  return (slot / kRun) * W + xcd * kRun + slot % kRun;
}

// Row order of K fed to the S^T mfma: swap bits 2 and 3 of the row index (an involution).
// With it, each lane half's accumulators of a 32-key block hold two runs of 8 consecutive
// keys, which is the order the P.V product takes its B operand in.
__device__ inline int rowperm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Asynchronous copy of 16 bytes per lane from global memory into LDS (lane i's bytes land
// at lds_dst + 16 i); completion is counted by vmcnt.
__device__ inline void load_lds16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const UF_GLOBAL void*)src, (UF_LDS void*)lds_dst, 16, 0, 0);
}

}  // namespace uf
