// gfx950 kernels of libuf: the block mask a head chooses for itself
// (Ultra Flash notes, key design 3, dynamic block-sparse causal attention).
//
// Every 128-token tile of the step's queries and of the visible keys is
// mean-pooled per head; a (query tile, key tile) pair is rated by the dot
// product of the two means; each (head, query tile) row keeps its local
// window (the key tiles overlapping its own key positions, widened by
// local_blocks tiles each side) plus the top_k best-rated other key tiles,
// equal ratings going to the lower tile index.
//
//   pool_kernel   one work-group per (tile, head): fp32 sum of the tile's
//                 bf16 rows (or E4M3 key rows, the mean then times the
//                 cache's k scale), divided by the row count.  HBM-bound: it
//                 reads q once and the visible K once.
//   select_kernel one work-group per (head, 4 query tiles): the 4 x n_kb
//                 ratings (fp32 fma chains over d in order) go to LDS as
//                 order-preserving 32-bit keys; then one wave per row finds
//                 the top_k-th largest candidate key by a bitwise search,
//                 counting with wave ballots, and writes the row's mask.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uf_device.h"
#include "uf_internal.h"

namespace uf {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 128;
constexpr int kRowsPerWg = 4;  // query tiles per selection work-group: one wave each

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Storage row of logical key j: anchor rows first, then the ring from its rotation.
__device__ inline int64_t key_row(const TopkParams& p, int j) {
  if (j < p.anchor_keys) return j;
  int r = j - p.anchor_keys + p.ring_rot;
  if (r >= p.ring_cap) r -= p.ring_cap;
  return (int64_t)p.ring_base + r;
}

// Work-groups [0, n_q_heads * n_qb) pool query tiles (tile-major, so
// neighbouring work-groups read neighbouring heads of the same tokens);
// the rest pool key tiles (head-major, neighbouring rows of one head).
template <int D>
__global__ void __launch_bounds__(kThreads) pool_kernel(TopkParams p) {
  constexpr int C = D / 8;           // 16-byte chunks per row
  constexpr int RP = kThreads / C;   // rows read side by side
  __shared__ float part[RP][D];
  const int r0 = threadIdx.x / C, c = threadIdx.x % C;
  const int q_jobs = p.n_q_heads * p.n_qb;
  const int b = blockIdx.x;
  const bool is_q = b < q_jobs;
  int head, tile, n_tok, n_rows;
  if (is_q) {
    tile = b / p.n_q_heads;
    head = b % p.n_q_heads;
    n_tok = p.n_q;
  } else {
    head = (b - q_jobs) / p.n_kb;
    tile = (b - q_jobs) % p.n_kb;
    n_tok = p.n_k;
  }
  n_rows = min(kTile, n_tok - tile * kTile);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = r0; r < n_rows; r += RP) {
    const int tok = tile * kTile + r;
    const int qtok = p.blk_h ? block_src_token(tok, p.blk_frames, p.blk_h, p.blk_w) : tok;
    if (!is_q && p.k_fp8) {
      // 8 E4M3 codes of channels 8c .. 8c + 7, decoded exactly to fp32
      const uint8_t* src = reinterpret_cast<const uint8_t*>(p.k) + (int64_t)head * p.kv_head_stride +
                           key_row(p, tok) * D + c * 8;
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
      const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
      const auto e = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
      const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
      acc[0] += a[0];
      acc[1] += a[1];
      acc[2] += b[0];
      acc[3] += b[1];
      acc[4] += e[0];
      acc[5] += e[1];
      acc[6] += f[0];
      acc[7] += f[1];
      continue;
    }
    const uint16_t* src = is_q ? p.q + (int64_t)qtok * p.q_stride_tok + (int64_t)head * p.q_stride_head
                               : p.k + (int64_t)head * p.kv_head_stride + key_row(p, tok) * D;
    const uint4 v = *reinterpret_cast<const uint4*>(src + c * 8);
    acc[0] += bf16_lo(v.x);
    acc[1] += bf16_hi(v.x);
    acc[2] += bf16_lo(v.y);
    acc[3] += bf16_hi(v.y);
    acc[4] += bf16_lo(v.z);
    acc[5] += bf16_hi(v.z);
    acc[6] += bf16_lo(v.w);
    acc[7] += bf16_hi(v.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RP; ++r) s += part[r][threadIdx.x];
    float mean = s / (float)n_rows;
    if (!is_q && p.k_fp8) mean *= p.k_scale;
    if (is_q)
      p.qbar[((int64_t)head * p.n_qb + tile) * D + threadIdx.x] = mean;
    else  // channel-major, so that the selection kernel reads neighbouring key tiles side by side
      p.kbar[((int64_t)head * D + threadIdx.x) * p.n_kb + tile] = mean;
  }
}

// Order-preserving map of a float to uint32 (larger float, larger key); -0 and +0 are one
// key.  Every finite rating maps to a key >= 1, so 0 can mark tiles that are not candidates.
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k > 1u ? k : 1u;
}


constexpr int kChanBatch = 32;

template <int D>
__global__ void __launch_bounds__(kThreads) select_kernel(TopkParams p) {
  extern __shared__ float lds[];
  const int n_kb = p.n_kb;
  const int n_kb_pad = (n_kb + 255) & ~255;  // rows padded with key 0 to whole groups of 4 x 64
  float* qs = lds;                                                   // [D][kRowsPerWg] query means
  uint32_t* keys = reinterpret_cast<uint32_t*>(lds + kRowsPerWg * D);  // [kRowsPerWg][n_kb_pad] rating keys
  const int head = blockIdx.x % p.n_q_heads;
  const int qb0 = (blockIdx.x / p.n_q_heads) * kRowsPerWg;
  const int g = head / (p.n_q_heads / p.n_kv_heads);
  for (int i = threadIdx.x; i < kRowsPerWg * D; i += kThreads) {
    const int r = i / D, c = i % D;
    qs[c * kRowsPerWg + r] = qb0 + r < p.n_qb ? p.qbar[((int64_t)head * p.n_qb + qb0 + r) * D + c] : 0.f;
  }
  __syncthreads();

  // Ratings.  Lanes take neighbouring key tiles, so each channel load is one coalesced row of
  // the channel-major key means; one LDS broadcast gives that channel of the 4 query means.
  static_assert(kRowsPerWg == 4, "one float4 of query means per channel");
  const float* kbar = p.kbar + (int64_t)g * D * n_kb;
  for (int kb = threadIdx.x; kb < n_kb_pad; kb += kThreads) {
    float a[kRowsPerWg] = {};
    if (kb < n_kb) {
      // kChanBatch channel loads in flight at a time: the loop is bound by L2 latency
      const float* col = kbar + kb;
      for (int c0 = 0; c0 < D; c0 += kChanBatch) {
        float kv[kChanBatch];
#pragma unroll
        for (int i = 0; i < kChanBatch; ++i) kv[i] = col[(int64_t)(c0 + i) * n_kb];
#pragma unroll
        for (int i = 0; i < kChanBatch; ++i) {
          const float4 qv = reinterpret_cast<const float4*>(qs)[c0 + i];
          a[0] = __builtin_fmaf(qv.x, kv[i], a[0]);
          a[1] = __builtin_fmaf(qv.y, kv[i], a[1]);
          a[2] = __builtin_fmaf(qv.z, kv[i], a[2]);
          a[3] = __builtin_fmaf(qv.w, kv[i], a[3]);
        }
      }
      if (p.scores) {
#pragma unroll
        for (int r = 0; r < kRowsPerWg; ++r)
          if (qb0 + r < p.n_qb) p.scores[((int64_t)head * p.n_qb + qb0 + r) * n_kb + kb] = a[r];
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWg; ++r) keys[r * n_kb_pad + kb] = kb < n_kb ? order_key(a[r]) : 0u;
  }
  __syncthreads();

  // Selection: one wave per query tile from here on; no barrier follows.  A wave's own LDS
  // accesses complete in order, so it may rewrite its row and read it back.
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qb = qb0 + w;
  if (qb >= p.n_qb) return;
  uint32_t* krow = keys + w * n_kb_pad;
  // local window: key tiles overlapping the tile's key positions, widened on both sides
  const int first = p.n_k - p.n_q + qb * kTile;
  const int last = p.n_k - p.n_q + min((qb + 1) * kTile, p.n_q) - 1;
  const int lo = max(0, first / kTile - p.local_blocks);
  const int hi = min(n_kb - 1, last / kTile + p.local_blocks);
  const int n_cand = n_kb - (hi - lo + 1);
  const int kk = min(p.top_k, n_cand);
  const bool keep_all = kk >= n_cand, keep_none = kk <= 0;
  for (int kb = lo + lane; kb <= hi; kb += 64) krow[kb] = 0u;  // window tiles are not candidates

  // T = the kk-th largest candidate key: the largest T with #{key >= T} >= kk (T >= 1).
  uint32_t T = 0xffffffffu;
  int need = 0;  // candidates equal to T that are kept (lowest tile indices first)
  if (!keep_all && !keep_none) {
    T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = T | (1u << bit);
      int cnt = 0;
      for (int base = lane; base < n_kb_pad; base += 256) {
        const uint32_t k0 = krow[base], k1 = krow[base + 64], k2 = krow[base + 128], k3 = krow[base + 192];
        cnt += __popcll(__ballot(k0 >= t)) + __popcll(__ballot(k1 >= t)) + __popcll(__ballot(k2 >= t)) +
               __popcll(__ballot(k3 >= t));
      }
      if (cnt >= kk) T = t;
    }
    int gt = 0;
    for (int base = lane; base < n_kb_pad; base += 256) {
      const uint32_t k0 = krow[base], k1 = krow[base + 64], k2 = krow[base + 128], k3 = krow[base + 192];
      gt += __popcll(__ballot(k0 > T)) + __popcll(__ballot(k1 > T)) + __popcll(__ballot(k2 > T)) +
            __popcll(__ballot(k3 > T));
    }
    need = kk - gt;
  }

  uint8_t* mrow = p.mask + ((int64_t)head * p.n_qb + qb) * n_kb;
  int taken = 0;
  const uint64_t below = (1ull << lane) - 1;
  for (int base = 0; base < n_kb_pad; base += 64) {
    const int kb = base + lane;
    const uint32_t key = krow[kb];
    const bool forced = kb >= lo && kb <= hi;
    bool keep = forced || (keep_all && key != 0u) || (!keep_none && key > T);
    const bool tie = !keep_all && !keep_none && key == T;
    const uint64_t ties = __ballot(tie);
    if (tie) keep = taken + __popcll(ties & below) < need;
    taken += __popcll(ties);
    if (kb < n_kb) mrow[kb] = keep ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_block_mask_topk(const TopkParams& p, int head_dim, hipStream_t stream) {
  const int pool_blocks = p.n_q_heads * p.n_qb + p.n_kv_heads * p.n_kb;
  const int select_blocks = p.n_q_heads * ((p.n_qb + kRowsPerWg - 1) / kRowsPerWg);
  const size_t lds = (size_t)kRowsPerWg * (head_dim + ((p.n_kb + 255) & ~255)) * sizeof(float);
  if (head_dim == 128) {
    hipLaunchKernelGGL(pool_kernel<128>, dim3(pool_blocks), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(select_kernel<128>, dim3(select_blocks), dim3(kThreads), lds, stream, p);
  } else {
    hipLaunchKernelGGL(pool_kernel<64>, dim3(pool_blocks), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(select_kernel<64>, dim3(select_blocks), dim3(kThreads), lds, stream, p);
  }
  return hipGetLastError();
}

}  // namespace uf
