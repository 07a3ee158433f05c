// Work items and key-tile walk shared by the bf16 and FP8 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uf_device.h"
#include "uf_internal.h"

namespace uf {

constexpr int kAttnTile = 128;  // keys per tile = block-mask tile = query rows per work-group

// What one lane of one work-group computes.  The grid enumerates (query block, split, head
// group) items, dealt to XCDs in windows (xcd_windowed); a work-group covers 128 / heads_per_wg
// queries of heads_per_wg query heads of one KV group, one 32-query row block per wave.
struct AttnItem {
  int split;   // part of the key range
  int q_tile;  // block-mask row (query tile)
  int head;    // this wave's query head
  int kvh;     // its KV head
  int qi;      // this lane's query row
  int qt;      // its token in q and out (differs from qi when the step is held in block order)
};

__device__ inline AttnItem attn_item(const AttnParams& p, int block, int n_blocks, int wave, int l32) {
  const int item = xcd_windowed(block, n_blocks);
  const int qblk = item % p.n_qblk;
  const int rest = item / p.n_qblk;
  const int hgrp = rest / p.splits;
  const int waves_per_head = 4 / p.heads_per_wg;
  const int q0 = qblk * (kAttnTile / p.heads_per_wg);
  AttnItem it;
  it.split = rest % p.splits;
  it.q_tile = q0 / kAttnTile;
  it.head = hgrp * p.heads_per_wg + wave / waves_per_head;
  it.kvh = (hgrp * p.heads_per_wg) / p.group;
  it.qi = q0 + (wave % waves_per_head) * 32 + l32;
  it.qt = p.blk_h && it.qi < p.n_q ? block_src_token(it.qi, p.blk_frames, p.blk_h, p.blk_w) : it.qi;
  return it;
}

// Storage row of logical key j: the anchor rows first, then the ring from its rotation.
__device__ inline int key_row(const AttnParams& p, int j) {
  if (j < p.anchor_keys) return j;
  int r = j - p.anchor_keys + p.ring_rot;
  if (r >= p.ring_cap) r -= p.ring_cap;
  return p.ring_base + r;
}

// First storage row of key tile kt when its 128 keys are 128 consecutive storage rows (a full
// tile that crosses neither the anchor/ring boundary nor the ring's wrap), else -1.
__device__ inline int contiguous_tile_rows(const AttnParams& p, int kt) {
  const int j0 = kt * kAttnTile;
  if (p.n_k - j0 < kAttnTile) return -1;
  if (j0 + kAttnTile <= p.anchor_keys) return j0;
  if (j0 < p.anchor_keys) return -1;
  int r = j0 - p.anchor_keys + p.ring_rot;
  if (r >= p.ring_cap) r -= p.ring_cap;
  return r + kAttnTile <= p.ring_cap ? p.ring_base + r : -1;
}

// The kept key tiles of one work item's mask row (every tile of its key range without a
// mask), in ascending order: 64 tiles at a time from a wave ballot over the mask row.  The
// tile returned is the same on every lane of the wave (and every wave of the work-group:
// heads_per_wg > 1 only with a mask shared by all heads).
struct KeyTiles {
  const uint8_t* mrow;
  int hi, w0;
  uint64_t bits;

  __device__ KeyTiles(const AttnParams& p, const AttnItem& it) {
    const int nkt = (p.n_k + kAttnTile - 1) / kAttnTile;
    const int lo = (int)(((int64_t)it.split * nkt) / p.splits);
    hi = (int)(((int64_t)(it.split + 1) * nkt) / p.splits);
    w0 = lo - 64;
    bits = 0;
    mrow = nullptr;
    if (p.mask) {
      const int mh = p.mask_heads == 1 ? 0 : it.head;
      mrow = p.mask + mh * p.mask_stride_head + (int64_t)it.q_tile * p.mask_stride_q;
    }
  }

  // next kept tile, or -1 when the row is exhausted
  __device__ int next(int lane) {
    while (bits == 0) {
      w0 += 64;
      if (w0 >= hi) return -1;
      if (mrow) {
        const int kt = w0 + lane;
        bits = __ballot(kt < hi && mrow[kt] != 0);
      } else {
        const int n = min(64, hi - w0);
        bits = n == 64 ? ~0ull : ((1ull << n) - 1ull);
      }
    }
    const int kt = w0 + __builtin_ctzll(bits);
    bits &= bits - 1;
    return __builtin_amdgcn_readfirstlane(kt);
  }
};

}  // namespace uf
