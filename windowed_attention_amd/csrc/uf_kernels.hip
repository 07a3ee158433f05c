// gfx950 kernels of libuf: rolling-cache append, chunk attention (bf16 MFMA,
// fp32 online softmax, block-mask tile skipping) and the split-KV combine.
//
// The attention operation is softmax(Q K^T / sqrt(d)) V over the cache's
// visible keys (FlashDecoder review, "Rolling KV cache", Eq. 4; HiStream
// summary, innovation 2 for the anchor), restricted to the kept 128x128
// tiles of an optional block mask (Ultra Flash notes, key design 3).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uf_attn_walk.h"
#include "uf_device.h"
#include "uf_internal.h"

namespace uf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves of 64
constexpr int kTile = 128;      // keys per tile = block-mask tile
// ---------------------------------------------------------------------------
// Append: token-major [t][h][c] -> head-major cache rows of the frame's slot.

__global__ void __launch_bounds__(kThreads) append_kernel(AppendParams p) {
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const uint16_t* __restrict__ src = p.src[which];
  uint16_t* __restrict__ dst = p.dst[which];
  const uint32_t chunks = (uint32_t)p.head_dim / 8;            // 16-byte chunks per row
  const uint32_t per_head = (uint32_t)p.n_tok * chunks;
  const uint32_t total = per_head * (uint32_t)p.n_heads;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const uint32_t h = i / per_head;
    const uint32_t r = i - h * per_head;
    const uint32_t t = r / chunks;
    const uint32_t c = r - t * chunks;
    const uint32_t f = t / (uint32_t)p.tokens_per_frame;
    const uint32_t tf = t - f * (uint32_t)p.tokens_per_frame;
    const int64_t gf = p.first_frame + f;
    const int64_t slot = gf < p.anchor_frames ? gf : p.anchor_frames + (gf - p.anchor_frames) % p.window_frames;
    const int64_t row = slot * p.tokens_per_frame + tf;
    // block order: the step's frames sit in consecutive slots and row t takes source token pi(t)
    const uint32_t ts = p.blk_h ? (uint32_t)block_src_token((int)t, p.n_tok / p.tokens_per_frame, p.blk_h, p.blk_w) : t;
    const uint4 val = *reinterpret_cast<const uint4*>(src + ts * p.src_stride_tok[which] +
                                                      h * p.src_stride_head[which] + c * 8);
    *reinterpret_cast<uint4*>(dst + ((int64_t)h * p.rows_total + row) * p.head_dim + c * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// Attention.
//
// Work-group: 4 waves, 128 (query, head) rows = 4 row blocks of 32 queries
// of one query head, one wave per row block; two work-groups share a CU.
// Per kept key tile (128 keys) the work-group stages K and V straight from
// global memory into LDS (global_load_lds, 16 bytes per lane, no register
// staging) and every wave computes its 32 rows against all 128 keys.  The
// LDS tile is single-buffered: while one work-group of a CU waits for its
// next tile, the other computes.
//
//   S^T = K . Q^T     mfma 32x32x16 bf16: A = K rows (LDS), B = Q^T (registers)
//   online softmax    fp32 per query (= per lane % 32); rescaling of the
//                     running output is skipped until the running max grows
//                     by more than 2^8 (exact: only the reference point moves);
//                     row sums of the bf16 probabilities with v_dot2
//   O^T += V^T . P^T  mfma 32x32x16: A = V^T read from the row-major V tile
//                     with the gfx950 LDS transpose read, B = P^T from the
//                     S^T registers
// K rows are fed to the S^T mfma in a permuted order (rowperm) so that each
// lane half's 8 keys of an S^T accumulator group are 8 consecutive keys:
// P^T then is the B operand of the PV mfma with no data movement.
//
// mfma_f32_32x32x16_bf16 operand layout (lane l, element e):
//   A[m = l % 32][k = 8*(l / 32) + e],  B[k = 8*(l / 32) + e][n = l % 32],
//   C[m = 8*(j / 4) + 4*(l / 32) + j % 4][n = l % 32] in accumulator j.
// ds_read_b64_tr_b16, per group of 16 lanes: lane i receives element i % 4
// of the 4-element (8-byte) reads of lanes 4r + i / 4, r = 0..3.
//
// LDS tiles are row-major (one key per row, head_dim contiguous) with the
// 16-byte chunks of every row permuted by an XOR swizzle (swz below).

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Chunk swizzle of LDS row r: its 16-byte chunk c is stored at position
// c ^ swz(r).  Chosen (exhaustively over linear maps of r mod 16) so that
// both the row-strided K reads (16 B per lane) and the transpose reads of V
// (8 B per lane) hit distinct banks with 32 or with 64 four-byte banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  const int r = row & 15;
  if constexpr (D == 128)
    return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 3 : 0);
  else
    return ((r & 1) ? 2 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 3 : 0);
}

constexpr int kAttnThreads = 256;  // 4 waves; two work-groups per CU

template <int D>
__global__ void __launch_bounds__(kAttnThreads, 2) attn_kernel(AttnParams p) {
  constexpr int NC = D / 16;            // 16-wide d chunks of the S^T mfma
  constexpr int ND = D / 32;            // 32-row d blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per LDS row
  constexpr int RB = D * 2;             // bytes per LDS row
  constexpr int TILE_B = kTile * RB;    // bytes per K (or V) tile
  constexpr int RPI = 64 / CPR;         // rows written by one wave-wide 16-byte load
  constexpr int NW = kAttnThreads / 64; // waves
  constexpr int NLD = kTile / RPI / NW; // such loads per wave, per tensor and tile
  __shared__ __attribute__((aligned(1024))) char smem[2 * TILE_B];  // [K tile][V tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int rb = wave;  // row block

  // ---- work item
  const AttnItem it = attn_item(p, blockIdx.x, gridDim.x, rb, l32);
  const int head = it.head, kvh = it.kvh, qi = it.qi, qt = it.qt;

  // ---- Q^T fragments (B operand), in registers for the whole key range
  bf16x8 qf[NC];
  {
    const bool ok = qi < p.n_q;
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(ok ? qt : 0) * p.q_stride_tok +
                       (int64_t)head * p.q_stride_head + 8 * half;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
      if (!ok) x = bf16x8{};
      qf[c] = x;
    }
  }
  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;  // reference max (raw score units) of this lane's query
  float l_run = 0.f;        // this lane half's sum of probabilities
  const float c2 = p.scale_log2;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)kvh * p.kv_head_stride;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)kvh * p.kv_head_stride;
  KeyTiles tiles(p, it);  // the kept key tiles, ascending

  // K and V of tile kt -> LDS (asynchronous; completion via vmcnt).  Lane
  // element offsets for a tile whose 128 keys are 128 consecutive storage
  // rows (every full tile that does not cross the anchor/ring boundary or
  // the ring's wrap): the tile is then one scalar base plus these offsets.
  uint32_t lane_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPI + lane / CPR;
    lane_off[i] = row * D + ((lane % CPR) ^ swz<D>(row)) * 8;
  }
  auto issue = [&](int kt) {
    const int j0 = kt * kTile;
    const int nvalid = min(kTile, p.n_k - j0);
    char* kd = smem + wave * NLD * 1024;
    char* vd = kd + TILE_B;
    const int r0 = contiguous_tile_rows(p, kt);
    if (r0 >= 0) {
      const __bf16* kt_base = kbase + (int64_t)r0 * D;
      const __bf16* vt_base = vbase + (int64_t)r0 * D;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        load_lds16(kt_base + lane_off[i], kd + i * 1024);
        load_lds16(vt_base + lane_off[i], vd + i * 1024);
      }
    } else {  // partial tile, or one that straddles the anchor/ring boundary or the wrap
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = (wave * NLD + i) * RPI + lane / CPR;
        const int chunk = (lane % CPR) ^ swz<D>(row);
        const int64_t off = (int64_t)key_row(p, j0 + min(row, nvalid - 1)) * D + chunk * 8;
        load_lds16(kbase + off, kd + i * 1024);
        load_lds16(vbase + off, vd + i * 1024);
      }
    }
  };
  // Per-lane LDS byte offsets of the fragment reads.  Every other term of an
  // address (key block, key chunk) is a multiple of 16 rows, leaves the
  // swizzle unchanged and goes into the instruction's immediate offset.
  uint32_t koff[NC];  // K rows for S^T: row 32*kb + rowperm(l32), chunk 2c + half
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int r = rowperm(l32);
    koff[c] = r * RB + (((2 * c + half) ^ swz<D>(r)) << 4);
  }
  uint32_t voff[ND][2];  // V rows for the transpose reads: key 16t + 8*half + 4*sub + (lane&15)/4
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int key = 8 * half + 4 * sub + ((lane & 15) >> 2);
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db][sub] = TILE_B + key * RB + ((((col >> 3) ^ swz<D>(key)) << 4) | ((col & 7) << 1));
    }
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v ones = {(__bf16)1.0f, (__bf16)1.0f};

  // one tile in LDS: S^T = K Q^T (4 blocks of 32 keys), softmax, O^T += V^T P^T
  auto compute = [&](int nvalid) {
    f32x16 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 a[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) a[kb] = *reinterpret_cast<const bf16x8*>(smem + koff[c] + 32 * kb * RB);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], qf[c], s[kb], 0, 0, 0);
    }
    // accumulator j of key block kb holds key 32*kb + 16*(j/8) + 8*half + j%8
    if (nvalid < kTile) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * kb + 16 * (j / 8) + 8 * half + (j % 8) >= nvalid) s[kb][j] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
    const float m_new = fmaxf(m_run, max_xor32(mx));
    const bool need = (m_new - m_run) * c2 > 8.f;  // lazy rescaling
    if (__ballot(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c2) : 1.f;
      if (need) m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i) o[i] *= alpha;
    }
    const float mc = m_run * c2;
    bf16x8 pb[8];  // P^T chunk t holds keys 16t + 8*half + e
    float lsum = l_run;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * hf + e], c2, -mc));
        const bf16x8 pk = __builtin_convertvector(pv, bf16x8);
        pb[2 * kb + hf] = pk;
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 0, 1), ones, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 2, 3), ones, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 4, 5), ones, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 6, 7), ones, lsum, false);
      }
    l_run = lsum;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bf16x8 a[ND];
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((UF_LDS i16x4*)(smem + voff[db][0] + 16 * t * RB));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((UF_LDS i16x4*)(smem + voff[db][1] + 16 * t * RB));
        a[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db], pb[t], o[db], 0, 0, 0);
    }
  };

  // ---- main loop: the other work-group on this CU computes while this one loads
  for (int kt = tiles.next(lane); kt >= 0; kt = tiles.next(lane)) {
    issue(kt);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // the tile is in LDS for every wave
    compute(min(kTile, p.n_k - kt * kTile));
    __syncthreads();  // every wave is done with the tile before the next one lands
  }

  // ---- epilogue.  O^T accumulator j of d block db holds d = 32*db + 8*(j/4) + 4*half + j%4.
  const float l = l_run + __shfl_xor(l_run, 32);
  if (qi >= p.n_q) return;
  if (p.splits == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)qt * p.o_stride_tok + (int64_t)head * p.o_stride_head;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g + 4 * half) = __builtin_convertvector(x, bf16x4);
      }
  } else {
    const int64_t row = ((int64_t)it.split * p.n_q + qt) * p.n_q_heads + head;
    float* wo = p.ws_o + row * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(wo + 32 * db + 8 * g + 4 * half) = x;
      }
    if (half == 0) {
      p.ws_ml[2 * row] = m_run * c2;  // -inf when this split saw no key
      p.ws_ml[2 * row + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV combine: out = sum_s w_s O_s / sum_s w_s l_s, w_s = 2^(m_s - max_s m_s).
// D / 8 lanes per (query, head) row, 8 channels each: two 16-byte loads per split and one
// 16-byte store per lane.

template <int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(CombineParams p) {
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPW = kThreads / LPR;     // rows per work-group
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / LPR;
  const int c0 = 8 * (threadIdx.x % LPR);
  const int64_t rows = (int64_t)p.n_q * p.n_q_heads;
  if (row >= rows) return;
  float mmax = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mmax = fmaxf(mmax, p.ws_ml[2 * (s * rows + row)]);
  f32x4 a0 = {}, a1 = {};
  float l = 0.f;
  if (mmax != -INFINITY) {
    for (int s = 0; s < p.splits; ++s) {
      const float* ml = p.ws_ml + 2 * (s * rows + row);
      const float w = __builtin_amdgcn_exp2f(ml[0] - mmax);
      l += w * ml[1];
      const f32x4* src = reinterpret_cast<const f32x4*>(p.ws_o + (s * rows + row) * D + c0);
      a0 += w * src[0];
      a1 += w * src[1];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int qi = (int)(row / p.n_q_heads), head = (int)(row % p.n_q_heads);
  __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)qi * p.o_stride_tok + (int64_t)head * p.o_stride_head + c0;
  const f32x8 x = {a0[0] * inv, a0[1] * inv, a0[2] * inv, a0[3] * inv, a1[0] * inv, a1[1] * inv, a1[2] * inv, a1[3] * inv};
  *reinterpret_cast<bf16x8*>(op) = __builtin_convertvector(x, bf16x8);
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const uint32_t total = (uint32_t)p.n_tok * (uint32_t)(p.head_dim / 8) * (uint32_t)p.n_heads;
  uint32_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(append_kernel, dim3(blocks, 2), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream) {
  const int items = p.n_qblk * p.n_hgrp * p.splits;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_kernel<128>, dim3(items), dim3(kAttnThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_kernel<64>, dim3(items), dim3(kAttnThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)p.n_q * p.n_q_heads;
  const int64_t rows_per_wg = kThreads / (head_dim / 8);
  const int blocks = (int)((rows + rows_per_wg - 1) / rows_per_wg);
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace uf
