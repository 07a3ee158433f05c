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
// queries of heads_per_wg query heads of one KV group, one 32-query row block per wave.  With
// an uneven two-part split (split_tile) the grid holds the long first parts of all items, then
// the short second parts, which start on the slots that free up (work-groups are dispatched in
// grid order as slots free up).
struct AttnItem {
  int split;   // part of the key range
  int q_tile;  // block-mask row (query tile)
  int head;    // this wave's query head
  int kvh;     // its KV head
  int qi;      // this lane's query row
  int qt;      // its token in q and out (differs from qi when the step is held in block order)
};

__device__ inline AttnItem attn_item(const AttnParams& p, int block, int n_blocks, int wave, int l32) {
  int item, split;
  if (p.split_tile) {
    const int per = n_blocks / 2;
    split = block >= per ? 1 : 0;
    item = xcd_windowed(block - split * per, per);
  } else {
    const int x = xcd_windowed(block, n_blocks);
    const int rest = x / p.n_qblk;
    split = rest % p.splits;
    item = x % p.n_qblk + (rest / p.splits) * p.n_qblk;
  }
  const int qblk = item % p.n_qblk;
  const int hgrp = item / p.n_qblk;
  const int waves_per_head = 4 / p.heads_per_wg;
  const int q0 = qblk * (kAttnTile / p.heads_per_wg);
  AttnItem it;
  it.split = split;
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
// tile returned is the same on every lane of the wave and every wave of the work-group.  With
// per-head masks and heads_per_wg > 1 the walk covers the union of the work-group's heads'
// rows, and `own` says whether the calling wave's head keeps the tile (its waves skip the
// others); otherwise `own` is always true.
struct KeyTiles {
  const uint8_t* mrow;     // first mask row of the walk (null: dense)
  const uint8_t* own_row;  // this wave's head's row
  int64_t row_stride;      // between the heads' rows of a union walk
  int n_rows;              // rows in the union (1 unless per-head masks are shared by the work-group)
  int hi, w0;
  uint64_t bits, own_bits;

  __device__ KeyTiles(const AttnParams& p, const AttnItem& it) {
    const int nkt = (p.n_k + kAttnTile - 1) / kAttnTile;
    int lo;
    if (p.split_tile) {
      lo = it.split ? p.split_tile : 0;
      hi = it.split ? nkt : p.split_tile;
    } else {
      lo = (int)(((int64_t)it.split * nkt) / p.splits);
      hi = (int)(((int64_t)(it.split + 1) * nkt) / p.splits);
    }
    w0 = lo - 64;
    bits = own_bits = 0;
    mrow = own_row = nullptr;
    row_stride = 0;
    n_rows = 1;
    if (p.mask) {
      const int64_t qoff = (int64_t)it.q_tile * p.mask_stride_q;
      if (p.mask_heads == 1) {
        mrow = own_row = p.mask + qoff;
      } else {
        const int h0 = it.head - it.head % p.heads_per_wg;  // the work-group's first head
        mrow = p.mask + h0 * p.mask_stride_head + qoff;
        own_row = p.mask + it.head * p.mask_stride_head + qoff;
        row_stride = p.mask_stride_head;
        n_rows = p.heads_per_wg;
      }
    }
  }

  // next kept tile, or -1 when the row is exhausted
  __device__ int next(int lane, bool& own) {
    while (bits == 0) {
      w0 += 64;
      if (w0 >= hi) return -1;
      if (mrow) {
        const int kt = w0 + lane;
        bool any = false;
        if (kt < hi)
          for (int r = 0; r < n_rows; ++r) any |= mrow[r * row_stride + kt] != 0;
        bits = __ballot(any);
        own_bits = n_rows == 1 ? bits : __ballot(kt < hi && own_row[kt] != 0);
      } else {
        const int n = min(64, hi - w0);
        bits = own_bits = n == 64 ? ~0ull : ((1ull << n) - 1ull);
      }
    }
    const int b = __builtin_ctzll(bits);
    bits &= bits - 1;
    own = __builtin_amdgcn_readfirstlane((int)((own_bits >> b) & 1)) != 0;
    return __builtin_amdgcn_readfirstlane(w0 + b);
  }
};

}  // namespace uf
