// Internal interface between the C ABI (uf_api.cpp) and the gfx950 kernels
// (uf_kernels.hip).  Plain structs passed to kernels by value.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace uf {

// Copy of n_tok tokens of K and V ([token][head][d], strided) into the
// head-major cache rows of their frames.
struct AppendParams {
  const uint16_t* src[2];      // k_new, v_new
  int64_t src_stride_tok[2];
  int64_t src_stride_head[2];
  uint16_t* dst[2];            // k_storage, v_storage
  int64_t rows_total;          // (A + W) * L rows per head
  int32_t n_tok;
  int32_t n_heads;
  int32_t head_dim;
  int32_t tokens_per_frame;    // L
  int32_t anchor_frames;       // A
  int32_t window_frames;       // W
  int64_t first_frame;         // global index of the first appended frame
  int32_t blk_h, blk_w;        // != 0: destination token t takes source token block_src_token(t)
};

// One attention step.  The grid is a flat list of work items
// (query block, head group, split) handed out XCD by XCD.
struct AttnParams {
  const uint16_t* q;
  int64_t q_stride_tok, q_stride_head;
  uint16_t* out;
  int64_t o_stride_tok, o_stride_head;
  const uint16_t* k;           // cache storage base
  const uint16_t* v;
  int64_t kv_head_stride;      // rows_total * head_dim
  int32_t n_q;                 // query rows
  int32_t n_k;                 // visible keys
  int32_t n_q_heads;
  int32_t group;               // Hq / Hkv
  int32_t heads_per_wg;        // 1, 2 or 4 query heads of one KV group per work-group
  int32_t n_qblk;              // query blocks of 128 / heads_per_wg rows
  int32_t n_hgrp;              // n_q_heads / heads_per_wg
  int32_t splits;              // key-range splits (1 = write out directly)
  int32_t split_tile;          // > 0: two uneven parts, key tiles [0, split_tile) and [split_tile, n_kb),
                               // every item's first part before any second part in the grid
  int32_t anchor_keys;         // logical keys [0, anchor_keys) are storage rows [0, anchor_keys)
  int32_t ring_base;           // storage row of ring slot 0 (= A * L)
  int32_t ring_cap;            // W * L
  int32_t ring_rot;            // recent key i is at ring_base + (i + ring_rot) mod ring_cap
  const uint8_t* mask;         // null = dense
  int32_t mask_heads;          // 1 or n_q_heads
  int32_t n_kb;                // key tiles of 128
  int64_t mask_stride_head, mask_stride_q;
  float scale_log2;            // log2(e) / sqrt(d)
  float* ws_o;                 // [splits][n_q][n_q_heads][d] unnormalised partial outputs
  float* ws_ml;                // [splits][n_q][n_q_heads][2]: running max (log2 units), sum
  int32_t blk_h, blk_w, blk_frames;  // != 0: query row i is token block_src_token(i) of q and out
  int32_t pipelined;           // head_dim 128: 1 = the software-pipelined loop, 0 = one sub-tile per step
};

// FP8 (E4M3) cache: the same append with each value quantized, code = E4M3(x * inv_scale),
// saturating at +-448; and the attention step on the FP8 storage.
struct AppendFp8Params {
  AppendParams a;              // dst[] point to uint8 storage; head_dim counts elements (bytes)
  float inv_scale[2];          // 1 / k_scale, 1 / v_scale
};

struct AttnFp8Params {
  AttnParams a;                // k, v point to uint8 storage; scale_log2 = log2(e) q_scale k_scale / sqrt(d)
  float q_inv_scale;           // q is quantized as E4M3(q * q_inv_scale)
  int q_e8m0;                  // 127 + E: the scores in log2 units are 2^E sum_c q8_c k8_c
  float v_scale;               // O = v_scale * sum_j P_j V8_j / sum_j P_j
};

struct CombineParams {
  const float* ws_o;
  const float* ws_ml;
  uint16_t* out;
  int64_t o_stride_tok, o_stride_head;
  int32_t n_q, n_q_heads, splits;
};

// Block-score top-k mask of one step: mean-pool the query tiles and the
// visible key tiles, score every (head, query tile, key tile) triple, keep the
// local window plus the top_k best other key tiles of each row.
struct TopkParams {
  const uint16_t* q;
  int64_t q_stride_tok, q_stride_head;
  const uint16_t* k;           // cache K storage base (bf16, or E4M3 bytes when k_fp8)
  int64_t kv_head_stride;      // rows_total * head_dim (elements)
  int32_t k_fp8;               // 1: K holds E4M3 codes, dequantized with k_scale
  float k_scale;
  int32_t n_q;                 // query rows (the newest n_q of the n_k keys)
  int32_t n_k;                 // visible keys
  int32_t n_q_heads, n_kv_heads;
  int32_t anchor_keys, ring_base, ring_cap, ring_rot;  // key order -> storage row, as in AttnParams
  int32_t n_qb, n_kb;          // query tiles, key tiles
  int32_t top_k;               // scored tiles kept per row beyond the local window
  int32_t local_blocks;        // tiles kept on each side of the diagonal tiles
  float* qbar;                 // workspace [n_q_heads][n_qb][d] tile means of q
  float* kbar;                 // workspace [n_kv_heads][d][n_kb] tile means of k, channel-major
  uint8_t* mask;               // [n_q_heads][n_qb][n_kb]
  float* scores;               // optional [n_q_heads][n_qb][n_kb]
  int32_t blk_h, blk_w, blk_frames;  // != 0: query row i is token block_src_token(i) of q
};

// Key tiles per row that the selection kernel holds in LDS (4 rows per work-group).
constexpr int kTopkMaxKeyTiles = 3072;

// Device memory of the allocation-free attention step: a file-scope array of
// kStaticScratchBytes per device, held until the process ends.  static_scratch() returns its
// device address on the current device (looked up once per device, then cached).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void** ptr);

hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream);
hipError_t launch_attention_d128(const AttnParams& p, hipStream_t stream);  // from launch_attention
hipError_t launch_attention_d64(const AttnParams& p, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream);
hipError_t launch_block_mask_topk(const TopkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_append_fp8(const AppendFp8Params& p, hipStream_t stream);
hipError_t launch_attention_fp8(const AttnFp8Params& p, int head_dim, hipStream_t stream);

}  // namespace uf
