// gfx950 kernels of libuf for a cache held in FP8 (E4M3): quantizing append and the
// attention step on FP8 matrix cores.
//
// Static FP8 quantization (FlashDecoder review, inference optimisations: statically
// calibrated FP8 for the matrix products): q, k and v are each quantized with one static
// scale, code = E4M3(x / scale) rounded to nearest even and saturated at +-448.  The step
// then computes softmax(Q K^T / sqrt(d)) V on the dequantized values:
//   S^T = K8 . Q8^T       mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulate);
//                         q is quantized with its scale rounded up so that
//                         log2(e) / sqrt(d) * q_scale * k_scale is a power of two 2^e, and 2^e
//                         is the Q operand's E8M0 scale: the scores come out in log2 units
//   P                     fp32 online softmax (lazy rescaling against an integer reference
//                         point m), E4M3(2^s / 2^m) from the scaled conversion (P <= 2^8 < 448)
//   O^T += V8^T . P8^T    the same mfma; V^T fragments come from the row-major V tile with
//                         the gfx950 LDS transpose read of bytes (ds_read_b64_tr_b8)
//   l                     one more mfma per 64 keys with an all-ones A operand, so the row
//                         sums add exactly the rounded probabilities the P.V product uses
//   out = v_scale * O / l
//
// Operand layout of the 32x32x64 FP8 mfma (checked on the GPU): lane l holds 32 bytes; A row
// m = l % 32 and B column n = l % 32 pair their bytes e in lane half h = l / 32 with the
// same k, i.e. C[m][n] = sum over (h, e) of A(lane m + 32h, byte e) * B(lane n + 32h, byte e);
// C is laid out as for the bf16 32x32 mfma.  ds_read_b64_tr_b8, per group of 16 lanes:
// lane i receives byte (i % 8) of the 8-byte reads of lanes 2k + i / 8, k = 0..7, as its
// byte k.  Reading with lane pairs (2k, 2k + 1) pointed at the same key row, 8 bytes apart,
// lane i then holds channel c0 + i of 8 consecutive keys.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uf_attn_walk.h"
#include "uf_device.h"
#include "uf_internal.h"

namespace uf {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 128;
constexpr float kMaxE4M3 = 448.f;

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline float sat(float x) { return fminf(fmaxf(x, -kMaxE4M3), kMaxE4M3); }

// four floats -> one dword of four E4M3 codes (byte i = value i), nearest even.  The first
// conversion writes the low half and keeps the high half of its `old` operand, which the
// second conversion overwrites; a's own bits serve as `old`, so no register has to be
// cleared first.
__device__ inline int pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// four floats divided by the power of two of `scale` (its exponent; v_cvt_scalef32) -> one
// dword of E4M3 codes, low byte first
__device__ inline int pack4_scaled(float a, float b, float c, float d, float scale) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  s16x2 w = __builtin_bit_cast(s16x2, __float_as_int(a));  // both halves are overwritten
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, scale, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, scale, true);
  return __builtin_bit_cast(int, w);
}

// eight bf16 (one 16-byte load) times s -> two dwords of E4M3 codes
__device__ inline void quant8(const uint4& v, float s, int& w0, int& w1) {
  w0 = pack4(sat(bf16_lo(v.x) * s), sat(bf16_hi(v.x) * s), sat(bf16_lo(v.y) * s), sat(bf16_hi(v.y) * s));
  w1 = pack4(sat(bf16_lo(v.z) * s), sat(bf16_hi(v.z) * s), sat(bf16_lo(v.w) * s), sat(bf16_hi(v.w) * s));
}

// ---------------------------------------------------------------------------
// Append: token-major bf16 [t][h][c] -> head-major E4M3 rows of the frame's slot; one
// thread per 16 channels of one (head, token).

__global__ void __launch_bounds__(kThreads) append_fp8_kernel(AppendFp8Params p) {
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const AppendParams& a = p.a;
  const uint16_t* __restrict__ src = a.src[which];
  uint8_t* __restrict__ dst = reinterpret_cast<uint8_t*>(a.dst[which]);
  const float s = p.inv_scale[which];
  const uint32_t chunks = (uint32_t)a.head_dim / 16;
  const uint32_t per_head = (uint32_t)a.n_tok * chunks;
  const uint32_t total = per_head * (uint32_t)a.n_heads;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const uint32_t h = i / per_head;
    const uint32_t r = i - h * per_head;
    const uint32_t t = r / chunks;
    const uint32_t c = r - t * chunks;
    const uint32_t f = t / (uint32_t)a.tokens_per_frame;
    const uint32_t tf = t - f * (uint32_t)a.tokens_per_frame;
    const int64_t gf = a.first_frame + f;
    const int64_t slot = gf < a.anchor_frames ? gf : a.anchor_frames + (gf - a.anchor_frames) % a.window_frames;
    const int64_t row = slot * a.tokens_per_frame + tf;
    const uint32_t ts = a.blk_h ? (uint32_t)block_src_token((int)t, a.n_tok / a.tokens_per_frame, a.blk_h, a.blk_w) : t;
    const uint16_t* sp = src + ts * a.src_stride_tok[which] + h * a.src_stride_head[which] + c * 16;
    const uint4 v0 = *reinterpret_cast<const uint4*>(sp);
    const uint4 v1 = *reinterpret_cast<const uint4*>(sp + 8);
    uint4 out;
    quant8(v0, s, reinterpret_cast<int&>(out.x), reinterpret_cast<int&>(out.y));
    quant8(v1, s, reinterpret_cast<int&>(out.z), reinterpret_cast<int&>(out.w));
    *reinterpret_cast<uint4*>(dst + ((int64_t)h * a.rows_total + row) * a.head_dim + c * 16) = out;
  }
}

// ---------------------------------------------------------------------------
// Attention.  Work-group and schedule as in the bf16 kernel: 4 waves, 128 (query, head)
// rows, one wave per 32-query row block, two work-groups per CU, K and V double-buffered in
// 64 KB of LDS.  FP8 tiles are half the bytes of bf16 ones, so the buffers hold whole
// 128-key tiles (the bf16 kernel's hold 64-key sub-tiles): the copy of the next kept tile
// runs under the computation of the current one.

// 16-byte chunk swizzle of LDS row r (rows of D bytes): chunk c sits at c ^ swz(r), which
// spreads both the 16-lane row-strided K reads and the 8-row transpose reads of V over
// all 64 banks.
template <int D>
__device__ __forceinline__ int swz8(int row) {
  constexpr int CPR = D / 16;
  constexpr int RPB = 256 / D;  // rows per 256 bytes of banks
  return (row / RPB) & (CPR - 1);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fp8_kernel(AttnFp8Params pp) {
  const AttnParams& p = pp.a;
  constexpr int NCH = D / 64;             // 64-deep d chunks of S = K Q^T
  constexpr int ND = D / 32;              // 32-row d blocks of O^T
  constexpr int CPR = D / 16;             // 16-byte chunks per LDS row
  constexpr int RB = D;                   // bytes per LDS row
  constexpr int TILE_B = kTile * RB;      // bytes per K (or V) tile
  constexpr int RPI = 64 / CPR;           // rows written by one wave-wide 16-byte load
  constexpr int NW = kThreads / 64;
  constexpr int NLD = kTile / RPI / NW;   // such loads per wave, per tensor and tile
  constexpr int BUF_B = 2 * TILE_B;       // one buffer: [K tile][V tile]
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int rb = wave;

  const AttnItem it = attn_item(p, blockIdx.x, gridDim.x, rb, l32);
  const int head = it.head, kvh = it.kvh, qi = it.qi, qt = it.qt;

  // ---- Q^T fragments (B operand): lane (query, half) holds channels 64c + 32 half .. +31
  i32x8 qf[NCH];
  {
    const bool ok = qi < p.n_q;
    const uint16_t* qp = p.q + (int64_t)(ok ? qt : 0) * p.q_stride_tok + (int64_t)head * p.q_stride_head + 32 * half;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      i32x8 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 v = *reinterpret_cast<const uint4*>(qp + 64 * c + 8 * j);
        if (!ok) v = make_uint4(0, 0, 0, 0);
        int w0, w1;
        quant8(v, pp.q_inv_scale, w0, w1);
        x[2 * j] = w0;
        x[2 * j + 1] = w1;
      }
      qf[c] = x;
    }
  }
  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = f32x16{};
  f32x16 lacc = f32x16{};    // every element: this lane's query's sum of rounded probabilities
  float m_run = -INFINITY;   // reference max (raw score units) of this lane's query
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + (int64_t)kvh * p.kv_head_stride;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + (int64_t)kvh * p.kv_head_stride;
  KeyTiles tiles(p, it);  // the kept key tiles, ascending

  uint32_t lane_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPI + lane / CPR;
    lane_off[i] = row * RB + (((lane % CPR) ^ swz8<D>(row)) << 4);
  }
  auto issue = [&](int kt, int buf) {
    const int j0 = kt * kTile;
    const int nvalid = min(kTile, p.n_k - j0);
    char* kd = smem + buf * BUF_B + wave * NLD * 1024;
    char* vd = kd + TILE_B;
    const int r0 = contiguous_tile_rows(p, kt);
    if (r0 >= 0) {
      const uint8_t* kt_base = kbase + (int64_t)r0 * RB;
      const uint8_t* vt_base = vbase + (int64_t)r0 * RB;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        copy16_async(kt_base, lane_off[i], kd + i * 1024);
        copy16_async(vt_base, lane_off[i], vd + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = (wave * NLD + i) * RPI + lane / CPR;
        const int chunk = (lane % CPR) ^ swz8<D>(row);
        const int64_t off = (int64_t)key_row(p, j0 + min(row, nvalid - 1)) * RB + chunk * 16;
        copy16_async(kbase + off, kd + i * 1024);
        copy16_async(vbase + off, vd + i * 1024);
      }
    }
  };
  // K fragment: row 32 kb + rowperm(l32), channels 64c + 32 half .. +31 = chunks 4c + 2 half + {0, 1};
  // 32 kb leaves the swizzle unchanged and goes into the immediate offset
  uint32_t koff[NCH][2];
  {
    const int r = rowperm(l32);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int i = 0; i < 2; ++i) koff[c][i] = r * RB + (((4 * c + 2 * half + i) ^ swz8<D>(r)) << 4);
  }
  // V transpose reads: lane (group g = lane / 16, s = lane % 16) points at key row
  // 8 half + s / 2 (+ 16 r + 64 t, immediates), channel 32 db + 16 (g & 1) + 8 (s & 1)
  uint32_t voff[ND];
  {
    const int s = lane & 15, g = lane >> 4;
    const int row = 8 * half + (s >> 1);
#pragma unroll
    for (int db = 0; db < ND; ++db)
      voff[db] = TILE_B + row * RB + (((2 * db + (g & 1)) ^ swz8<D>(row)) << 4) + 8 * (s & 1);
  }
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0

  auto mfma8 = [](const i32x8& a, const i32x8& b, const f32x16& c) -> f32x16 {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  };
  // S = K Q^T with the power of two 2^E of q's scale applied to the Q operand (E8M0 scale
  // 127 + E): the accumulators then hold the scores in log2 units exactly, with no multiply
  const int q_e8m0 = pp.q_e8m0;
  auto mfma8q = [q_e8m0](const i32x8& a, const i32x8& b, const f32x16& c) -> f32x16 {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, q_e8m0);
  };

  auto compute = [&](int nvalid, int buf) {
    const char* tb = smem + buf * BUF_B;
    f32x16 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = f32x16{};
    // MFMA m = 4c + kb takes the K fragment of d chunk c, key block kb.  Fragments are read two
    // MFMAs ahead (a ring of three in registers), and the schedule below keeps that order: left
    // to itself the compiler waits for each fragment right before its MFMA.
    constexpr int NS = 4 * NCH;
    auto kfrag = [&](int m) {
      const int c = m / 4, kb = m % 4;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(tb + koff[c][0] + 32 * kb * RB);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(tb + koff[c][1] + 32 * kb * RB);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    i32x8 ka[3];
    ka[0] = kfrag(0);
    ka[1] = kfrag(1);
#pragma unroll
    for (int m = 0; m < NS; ++m) {
      if (m + 2 < NS) ka[(m + 2) % 3] = kfrag(m + 2);
      s[m % 4] = mfma8q(ka[m % 3], qf[m / 4], s[m % 4]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the fragments of MFMAs 0 and 1
#pragma unroll
    for (int m = 0; m < NS; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA m
      if (m + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the fragment of MFMA m + 2
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
    // Lazy rescaling against an integer reference point m_run (log2 units): it moves, to the
    // floor of the running max, only when the max has grown by more than 8, so P stays below
    // 2^8 (E4M3 holds 448) and every rescaling factor is an exact power of two.
    const float m_new = fmaxf(m_run, max_xor32(mx));
    const bool need = m_new - m_run > 8.f;
    if (__ballot(need)) {
      const float ref = need ? floorf(m_new) : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - ref);  // 0 for the first tile (-inf)
      m_run = ref;
      lacc *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i) o[i] *= alpha;
    }
    // P = E4M3(2^(s - m_run)).  While |m_run| <= 96 the conversion divides by 2^m_run itself
    // (v_cvt_scalef32, exact on the fp32 value 2^s: s <= m_run + 8 cannot overflow, and where 2^s
    // leaves the normal range the code is 0 either way), so no subtraction per score is needed.
    const bool scaled = __ballot(!(fabsf(m_run) <= 96.f)) == 0;
    // 2^m_run (m_run clamped to the range the scaled path is taken in, so that the conversion
    // to an integer is defined whatever m_run holds)
    const float ref_scale = __int_as_float(((int)fminf(fmaxf(m_run, -96.f), 96.f) + 127) << 23);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // P^T (B operand) of keys 64t .. 64t + 63: byte 8r + k of lane half h is key
      // 64t + 16r + 8h + k, i.e. dword w packs accumulators 4(w & 3) .. +3 of key block 2t + w / 4
      i32x8 pf;
      if (scaled) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const f32x16& blk = s[2 * t + (w >> 2)];
          const int j = 4 * (w & 3);
          pf[w] = pack4_scaled(__builtin_amdgcn_exp2f(blk[j]), __builtin_amdgcn_exp2f(blk[j + 1]),
                               __builtin_amdgcn_exp2f(blk[j + 2]), __builtin_amdgcn_exp2f(blk[j + 3]), ref_scale);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const f32x16& blk = s[2 * t + (w >> 2)];
          const int j = 4 * (w & 3);
          pf[w] = pack4(__builtin_amdgcn_exp2f(blk[j] - m_run), __builtin_amdgcn_exp2f(blk[j + 1] - m_run),
                        __builtin_amdgcn_exp2f(blk[j + 2] - m_run), __builtin_amdgcn_exp2f(blk[j + 3] - m_run));
        }
      }
      lacc = mfma8(ones, pf, lacc);
      // V^T fragments one d block ahead of their MFMA (the same ordering trick as for K)
      auto vfrag = [&](int db) {
        i32x8 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (UF_LDS i32x2*)(tb + voff[db] + (64 * t + 16 * r) * RB));
          a[2 * r] = v[0];
          a[2 * r + 1] = v[1];
        }
        return a;
      };
      i32x8 va[3];
      va[0] = vfrag(0);
      if (ND > 1) va[1] = vfrag(1);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        if (db + 2 < ND) va[(db + 2) % 3] = vfrag(db + 2);
        o[db] = mfma8(va[db % 3], pf, o[db]);
      }
      // reads of d blocks 0 and 1, the row-sum MFMA and the MFMA of block 0, then per block the
      // reads two ahead and its MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, ND > 1 ? 8 : 4, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
#pragma unroll
      for (int db = 1; db < ND; ++db) {
        if (db + 1 < ND) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      }
    }
  };

  // Tile i sits in buffer i % 2.  The barrier at the top of step i publishes tile i (every
  // wave has waited for its own copies) and also shows that every wave has finished tile
  // i - 1, whose buffer the copy of tile i + 1 then overwrites.
  bool own, own_next;
  int kt = tiles.next(lane, own);
  int buf = 0;
  if (kt >= 0) issue(kt, 0);
  while (kt >= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int kn = tiles.next(lane, own_next);
    if (kn >= 0) issue(kn, buf ^ 1);
    if (own) compute(min(kTile, p.n_k - kt * kTile), buf);
    kt = kn;
    own = own_next;
    buf ^= 1;
  }

  // ---- epilogue.  O^T accumulator j of d block db holds d = 32*db + 8*(j/4) + 4*half + j%4.
  const float l = lacc[0];
  if (qi >= p.n_q) return;
  if (p.splits == 1) {
    const float inv = l > 0.f ? pp.v_scale / l : 0.f;
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
        f32x4 x = {o[db][4 * g] * pp.v_scale, o[db][4 * g + 1] * pp.v_scale, o[db][4 * g + 2] * pp.v_scale,
                   o[db][4 * g + 3] * pp.v_scale};
        *reinterpret_cast<f32x4*>(wo + 32 * db + 8 * g + 4 * half) = x;
      }
    if (half == 0) {
      p.ws_ml[2 * row] = m_run;  // log2 units; -inf when this split saw no key
      p.ws_ml[2 * row + 1] = l;
    }
  }
}

}  // namespace

hipError_t launch_append_fp8(const AppendFp8Params& p, hipStream_t stream) {
  const uint32_t total = (uint32_t)p.a.n_tok * (uint32_t)(p.a.head_dim / 16) * (uint32_t)p.a.n_heads;
  uint32_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(append_fp8_kernel, dim3(blocks, 2), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention_fp8(const AttnFp8Params& p, int head_dim, hipStream_t stream) {
  const int items = p.a.n_qblk * p.a.n_hgrp * p.a.splits;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_fp8_kernel<128>, dim3(items), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fp8_kernel<64>, dim3(items), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace uf
