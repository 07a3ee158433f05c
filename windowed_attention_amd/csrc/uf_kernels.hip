// gfx950 kernels of libuf: rolling-cache append, the launch of the bf16 chunk attention
// kernel (bf16 MFMA, fp32 online softmax, block-mask tile skipping; uf_attn_bf16.h, its
// instances in uf_attn_d128.hip and uf_attn_d64.hip) and the split-KV combine.
//
// The attention operation is softmax(Q K^T / sqrt(d)) V over the cache's
// visible keys (FlashDecoder review, "Rolling KV cache", Eq. 4; HiStream
// summary, innovation 2 for the anchor), restricted to the kept 128x128
// tiles of an optional block mask (Ultra Flash notes, key design 3).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "uf_attn_walk.h"
#include "uf_device.h"
#include "uf_internal.h"

namespace uf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves of 64
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

// ---------------------------------------------------------------------------
// Scratch of the allocation-free attention step (split partials), one copy per device.  In
// host code `scratch` names a host-side stand-in, not the device array: its device address
// comes from hipGetSymbolAddress, taken once per device with that device current, and only
// that address is ever passed to a kernel.

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const uint32_t total = (uint32_t)p.n_tok * (uint32_t)(p.head_dim / 8) * (uint32_t)p.n_heads;
  uint32_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(append_kernel, dim3(blocks, 2), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_attention_d128(p, stream) : launch_attention_d64(p, stream);
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
