// Device helpers shared by the gfx950 kernels of libuf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define UF_LDS __attribute__((address_space(3)))

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

// Maximum of x over lanes l and l ^ 32 (the two halves of a wave).  One v_permlane32_swap
// of x with itself leaves, in every lane, x of lane l in one result and x of lane l ^ 32 in
// the other: lanes 0-31 keep their own value and receive lane l + 32's, lanes 32-63 receive
// lane l - 32's and keep their own.
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Global -> LDS copy of 16 bytes per lane (lane i's bytes land at lds_dst + 16 i), as inline
// asm: the instruction has no register result, and written this way the compiler does not
// take it for an LDS store that every later LDS read must wait for, which would hold the
// reads of the current tile until the next tile's copy has landed.  The callers wait for
// the copies themselves (s_waitcnt vmcnt(0) before the barrier that publishes a tile).
// The LDS address goes in M0, which the compiler reserves: each statement saves M0 in a
// scratch SGPR and restores it after the instruction has issued.
__device__ inline void copy16_async(const void* src, void* lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(UF_LDS void*)lds_dst);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds), "v"(src)
               : "memory");
}
// The same from a wave-uniform base plus a 32-bit per-lane byte offset (the scalar-base
// form of the instruction: no per-lane 64-bit address arithmetic).
__device__ inline void copy16_async(const void* base, uint32_t off, void* lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(UF_LDS void*)lds_dst);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds), "v"(off), "s"(sb)
               : "memory");
}


// Raster token (frame f, row y, column x -> (f H + y) W + x) at position i of a step's
// block order, for F frames of an H x W grid (Ultra Flash notes, key design 3: (2,8,8)
// spatio-temporal blocks): first the frame pairs' full (2,8,8) blocks (pair by pair, blocks
// row-major, inside a block frame, row, column), then the odd last frame's full 8x8 patches,
// then every token outside a full block or patch in raster order.
__device__ inline int block_src_token(int i, int F, int H, int W) {
  const int hb = H >> 3, wb = W >> 3, nb = hb * wb;
  const int region_a = (F >> 1) * nb * 128;
  if (i < region_a) {
    const int p = i / (nb * 128), rem = i - p * nb * 128;
    const int b = rem >> 7, w = rem & 127;
    const int y = 8 * (b / wb) + ((w >> 3) & 7), x = 8 * (b % wb) + (w & 7);
    return ((2 * p + (w >> 6)) * H + y) * W + x;
  }
  i -= region_a;
  const int region_b = (F & 1) * nb * 64;
  if (i < region_b) {
    const int b = i >> 6, w = i & 63;
    return ((F - 1) * H + 8 * (b / wb) + (w >> 3)) * W + 8 * (b % wb) + (w & 7);
  }
  i -= region_b;
  const int edge = H * W - 64 * nb;           // tokens of a frame outside full blocks
  const int f = i / edge, k = i - f * edge;
  const int right = W - 8 * wb;               // columns right of the last full block
  const int beside = 8 * hb * right;          // leftover tokens in the block rows
  int y, x;
  if (k < beside) {
    y = k / right;
    x = 8 * wb + (k - y * right);
  } else {
    const int k2 = k - beside;
    y = 8 * hb + k2 / W;
    x = k2 - (k2 / W) * W;
  }
  return (f * H + y) * W + x;
}

}  // namespace uf
