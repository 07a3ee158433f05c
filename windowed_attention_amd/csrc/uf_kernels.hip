// gfx950 kernels of libuf: rolling-cache append, chunk attention (bf16 MFMA,
// fp32 online softmax, block-mask tile skipping) and the split-KV combine.
//
// The attention operation is softmax(Q K^T / sqrt(d)) V over the cache's
// visible keys (FlashDecoder review, "Rolling KV cache", Eq. 4; HiStream
// summary, innovation 2 for the anchor), restricted to the kept 128x128
// tiles of an optional block mask (Ultra Flash notes, key design 3).
#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr int kXcds = 8;        // MI355X: 8 XCDs, work-groups dealt round-robin

// Work-group b is dispatched to XCD b % 8.  Renumber so that each XCD gets
// one contiguous run of work items (neighbouring query blocks of the same
// head), which then share K/V tiles in that XCD's L2.
__device__ inline int xcd_contiguous(int b, int n) {
  const int per = n / kXcds, extra = n % kXcds;
  const int xcd = b % kXcds, slot = b / kXcds;
  return xcd * per + min(xcd, extra) + slot;
}

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
    const uint4 val = *reinterpret_cast<const uint4*>(src + t * p.src_stride_tok[which] +
                                                      h * p.src_stride_head[which] + c * 8);
    *reinterpret_cast<uint4*>(dst + ((int64_t)h * p.rows_total + row) * p.head_dim + c * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// Attention.
//
// Work-group: 4 waves, 128 (query, head) rows.  Each wave owns 32 queries of
// one query head.  Per key tile of 128 keys:
//   S^T = K . Q^T   mfma 32x32x16 bf16: A = K rows from LDS, B = Q^T in registers
//   online softmax  fp32, per query = per lane (query = lane % 32), the two
//                   lane halves hold different keys of the same query
//   O^T += V^T . P^T  mfma 32x32x16: A = V^T from LDS (stored transposed),
//                   B = P^T straight from the S^T registers.
// K rows are fed to the S^T mfma in a permuted order (rowperm) so that the
// 16 keys of each S^T register group that a lane half holds are 8
// consecutive keys: P^T then serves as the B operand of the PV mfma with no
// data movement.
//
// mfma_f32_32x32x16_bf16 operand layout (lane l, element e):
//   A[m = l % 32][k = 8*(l / 32) + e],  B[k = 8*(l / 32) + e][n = l % 32],
//   C[m = 8*(j / 4) + 4*(l / 32) + j % 4][n = l % 32] in accumulator j.

__device__ inline int rowperm(int m) {  // swap bits 2 and 3 (an involution)
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D>
struct AttnSmem {
  static constexpr int kStr = D + 8;        // K row stride (elements), +16 B against bank conflicts
  static constexpr int vStr = kTile + 8;    // V^T row stride (one row per d)
  __bf16 k[kTile * kStr];
  __bf16 vt[D * vStr];
};

template <int D>
__global__ void __launch_bounds__(kThreads, 1) attn_kernel(AttnParams p) {
  constexpr int NC = D / 16;  // 16-wide d chunks of the S^T mfma
  constexpr int ND = D / 32;  // 32-row d blocks of O^T
  constexpr int kStr = AttnSmem<D>::kStr;
  constexpr int vStr = AttnSmem<D>::vStr;
  __shared__ AttnSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  // ---- work item
  const int item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int qblk = item % p.n_qblk;
  const int rest = item / p.n_qblk;
  const int split = rest % p.splits;
  const int hgrp = rest / p.splits;
  const int waves_per_head = 4 / p.heads_per_wg;
  const int qpw = kTile / p.heads_per_wg;                     // queries per work-group
  const int head = hgrp * p.heads_per_wg + wave / waves_per_head;
  const int q0 = qblk * qpw;
  const int qi = q0 + (wave % waves_per_head) * 32 + l32;     // this lane's query row
  const int kvh = head / p.group;
  const int q_tile = q0 / kTile;                              // block-mask row

  // ---- Q^T fragments (B operand), kept in registers for the whole key range
  bf16x8 qf[NC];
  {
    const bool ok = qi < p.n_q;
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)(ok ? qi : 0) * p.q_stride_tok +
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
  float m_run = -INFINITY;  // running max of raw scores for this lane's query
  float l_run = 0.f;        // this lane half's partial sum of probabilities
  const float c2 = p.scale_log2;

  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)kvh * p.kv_head_stride;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)kvh * p.kv_head_stride;

  // storage row of logical key j
  auto key_row = [&](int j) -> int {
    if (j < p.anchor_keys) return j;
    int r = j - p.anchor_keys + p.ring_rot;
    if (r >= p.ring_cap) r -= p.ring_cap;
    return p.ring_base + r;
  };

  const int nkt = (p.n_k + kTile - 1) / kTile;
  const int kt_lo = (int)(((int64_t)split * nkt) / p.splits);
  const int kt_hi = (int)(((int64_t)(split + 1) * nkt) / p.splits);

  const uint8_t* mrow = nullptr;
  if (p.mask) {
    const int mh = p.mask_heads == 1 ? 0 : head;  // heads_per_wg > 1 only with a shared mask
    mrow = p.mask + mh * p.mask_stride_head + (int64_t)q_tile * p.mask_stride_q;
  }

  for (int w0 = kt_lo; w0 < kt_hi; w0 += 64) {
    uint64_t bits;
    if (mrow) {
      const int kt = w0 + lane;
      const bool keep = kt < kt_hi && mrow[kt] != 0;
      bits = __ballot(keep);
    } else {
      const int n = min(64, kt_hi - w0);
      bits = n == 64 ? ~0ull : ((1ull << n) - 1ull);
    }
    while (bits) {
      const int kt = w0 + __builtin_ctzll(bits);
      bits &= bits - 1;
      const int j0 = kt * kTile;
      const int nvalid = min(kTile, p.n_k - j0);

      __syncthreads();  // previous tile's LDS reads are done
      // ---- K tile -> LDS, row-major [key][d]
      {
        constexpr int cpr = D / 8;             // 16-byte chunks per row
        constexpr int rpp = kThreads / cpr;    // rows per pass
        const int c8 = tid % cpr;
#pragma unroll
        for (int r = tid / cpr; r < kTile; r += rpp) {
          uint4 val = make_uint4(0, 0, 0, 0);
          if (r < nvalid) val = *reinterpret_cast<const uint4*>(kbase + (int64_t)key_row(j0 + r) * D + c8 * 8);
          *reinterpret_cast<uint4*>(&sm.k[r * kStr + c8 * 8]) = val;
        }
      }
      // ---- V tile -> LDS, transposed [d][key]
      {
        const int r = tid % kTile;            // key within the tile
        const bool ok = r < nvalid;
        const __bf16* vrow = vbase + (int64_t)(ok ? key_row(j0 + r) : 0) * D;
#pragma unroll
        for (int c8 = tid / kTile; c8 < D / 8; c8 += kThreads / kTile) {
          bf16x8 val = *reinterpret_cast<const bf16x8*>(vrow + c8 * 8);
          if (!ok) val = bf16x8{};
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.vt[(c8 * 8 + e) * vStr + r] = val[e];
        }
      }
      __syncthreads();

      // ---- S^T = K Q^T for 4 blocks of 32 keys
      f32x16 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x16{};
        const __bf16* krow = &sm.k[(32 * kb + rowperm(l32)) * kStr + 8 * half];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * c);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
        }
      }
      // S^T accumulator j of block kb holds key 32*kb + 16*(j/8) + 8*half + j%8
      if (nvalid < kTile) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * kb + 16 * (j / 8) + 8 * half + (j % 8) >= nvalid) s[kb][j] = -INFINITY;
      }

      // ---- online softmax (fp32)
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i) o[i] *= alpha;
      const float mc = m_new * c2;

      bf16x8 pb[8];  // P^T for 8 chunks of 16 keys: chunk t holds keys 16t + 8*half + e
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x8 pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = __builtin_amdgcn_exp2f(s[kb][8 * hf + e] * c2 - mc);
            l_run += x;
            pv[e] = x;
          }
          pb[2 * kb + hf] = __builtin_convertvector(pv, bf16x8);
        }
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const __bf16* vrow = &sm.vt[(32 * db + l32) * vStr + 8 * half];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + 16 * t);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], o[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue.  O^T accumulator j of d-block db holds d = 32*db + 8*(j/4) + 4*half + j%4.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi >= p.n_q) return;
  if (p.splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)qi * p.o_stride_tok + (int64_t)head * p.o_stride_head;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g + 4 * half) = __builtin_convertvector(x, bf16x4);
      }
  } else {
    const int64_t row = ((int64_t)split * p.n_q + qi) * p.n_q_heads + head;
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
      p.ws_ml[2 * row + 1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV combine: out = sum_s w_s O_s / sum_s w_s l_s, w_s = 2^(m_s - max_s m_s).
// One wave per (query, head) row.

template <int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.n_q * p.n_q_heads;
  if (row >= rows) return;
  float mmax = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mmax = fmaxf(mmax, p.ws_ml[2 * (s * rows + row)]);
  constexpr int PER = D / 64;  // d values per lane
  float acc[PER] = {};
  float l = 0.f;
  if (mmax != -INFINITY) {
    for (int s = 0; s < p.splits; ++s) {
      const float w = __builtin_amdgcn_exp2f(p.ws_ml[2 * (s * rows + row)] - mmax);
      l += w * p.ws_ml[2 * (s * rows + row) + 1];
      const float* src = p.ws_o + (s * rows + row) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += w * src[lane * PER + i];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int qi = (int)(row / p.n_q_heads), head = (int)(row % p.n_q_heads);
  __bf16* op = reinterpret_cast<__bf16*>(p.out) + (int64_t)qi * p.o_stride_tok + (int64_t)head * p.o_stride_head;
#pragma unroll
  for (int i = 0; i < PER; ++i) op[lane * PER + i] = (__bf16)(acc[i] * inv);
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
    hipLaunchKernelGGL(attn_kernel<128>, dim3(items), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_kernel<64>, dim3(items), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)p.n_q * p.n_q_heads;
  const int blocks = (int)((rows + 3) / 4);
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace uf
