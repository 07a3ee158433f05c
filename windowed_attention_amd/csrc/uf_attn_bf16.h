// The bf16 attention kernel of libuf (gfx950): chunk attention with bf16 MFMA, fp32 online
// softmax and block-mask tile skipping over the rolling cache (FlashDecoder review, "Rolling
// KV cache", Eq. 4; HiStream summary, innovation 2 for the anchor; Ultra Flash notes, key
// design 3 for the block mask).  Included by uf_attn_d128.hip and uf_attn_d64.hip, each built
// with its own scheduling option; each has its own copy of the template, with internal
// linkage.
#pragma once

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

constexpr int kAttnTileKeys = 128;  // keys per tile = block-mask tile

// ---------------------------------------------------------------------------
// Attention.
//
// Work-group: 4 waves, 128 (query, head) rows = 4 row blocks of 32 queries
// of one query head, one wave per row block; two work-groups share a CU.
// Each kept key tile (128 keys) is taken as two 64-key sub-tiles.  The
// work-group stages K and V of a sub-tile straight from global memory into
// LDS (global_load_lds, 16 bytes per lane, no register staging) and every
// wave computes its 32 rows against its 64 keys.  K and V are double-
// buffered: two sub-tile buffers of 32 KB, the 64 KB one 128-key tile would
// take, so that two work-groups still share a CU.  The copy of sub-tile
// j + 1 goes out during the S MFMAs of sub-tile j and is waited for at the
// end of step j.
//
// Two loops (PIPE):
//   * one sub-tile per step: S, softmax and P.V of sub-tile j, then a barrier;
//   * software-pipelined (head_dim 128, long key walks): step j multiplies S of
//     sub-tile j + 1 while it exponentiates the scores of sub-tile j, then
//     P.V of sub-tile j, then takes the maximum of the new scores, so that
//     each wave has exponentials to issue beside both of its MFMA blocks.  K
//     is copied two sub-tiles ahead and V one ahead, in the same 64 KB.
// Both take the same arithmetic in the same order, so their outputs are
// identical bit for bit.
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

constexpr int kAttnThreads = 256;  // 4 waves
// Work-groups per CU the register allocation is held to: two at d = 128 (LDS 64 KB each); four
// at d = 64 (LDS 32 KB, 128 registers per wave: decoder-XL and refine-XL +3% over three).
template <int D>
constexpr int attn_wgs_per_cu() { return D == 64 ? 4 : 2; }

constexpr int kSub = 64;  // keys per sub-tile: two per key tile

template <int D, bool PIPE>
__global__ void __launch_bounds__(kAttnThreads, attn_wgs_per_cu<D>()) attn_kernel(AttnParams p) {
  constexpr int NC = D / 16;            // 16-wide d chunks of the S^T mfma
  constexpr int ND = D / 32;            // 32-row d blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per LDS row
  constexpr int RB = D * 2;             // bytes per LDS row
  constexpr int SUB_B = kSub * RB;      // bytes per K (or V) sub-tile
  constexpr int RPI = 64 / CPR;         // rows written by one wave-wide 16-byte load
  constexpr int NLD = 16 / RPI;         // such loads per wave, per tensor and sub-tile (16 rows)
  __shared__ __attribute__((aligned(1024))) char smem[4 * SUB_B];  // [K0][V0][K1][V1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int rb = wave;

  const AttnItem it = attn_item(p, blockIdx.x, gridDim.x, rb, l32);
  const int head = it.head, kvh = it.kvh, qi = it.qi, qt = it.qt;

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
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = p.scale_log2;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)kvh * p.kv_head_stride;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)kvh * p.kv_head_stride;
  KeyTiles tiles(p, it);

  // This wave copies rows 16 wave .. + 15 of every K and V sub-tile.
  const int row0 = 16 * wave;
  uint32_t lane_off[NLD];  // byte offsets within a sub-tile of 64 consecutive storage rows
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = row0 + i * RPI + lane / CPR;
    lane_off[i] = (uint32_t)(row * D + ((lane % CPR) ^ swz<D>(row)) * 8) * 2u;
  }
  // Byte offsets, from the head's base, of this wave's copy rows of the sub-tile starting at
  // key j0 (the same for K and V); j0 < 0 gives row 0 of the head, a harmless copy into a
  // buffer that is not read again.  (The host keeps a head's storage under 4 GB.)
  auto copy_offsets = [&](int j0, uint32_t (&off)[NLD]) {
    int r0 = -1;
    if (j0 >= 0 && p.n_k - j0 >= kSub) {
      if (j0 + kSub <= p.anchor_keys) {
        r0 = j0;
      } else if (j0 >= p.anchor_keys) {
        int r = j0 - p.anchor_keys + p.ring_rot;
        if (r >= p.ring_cap) r -= p.ring_cap;
        if (r + kSub <= p.ring_cap) r0 = p.ring_base + r;
      }
    }
    if (r0 >= 0) {
      const uint32_t b = (uint32_t)r0 * (uint32_t)RB;
#pragma unroll
      for (int i = 0; i < NLD; ++i) off[i] = b + lane_off[i];
    } else if (j0 >= 0) {
      const int nvalid = min(kSub, p.n_k - j0);
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = row0 + i * RPI + lane / CPR;
        const int chunk = (lane % CPR) ^ swz<D>(row);
        off[i] = ((uint32_t)key_row(p, j0 + min(row, nvalid - 1)) * D + chunk * 8) * 2u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) off[i] = (uint32_t)(lane % CPR) * 16u;
    }
  };
  // K rows for S^T: row 32 kb + rowperm(l32), chunk 2c + half at position (half ^ swz) ^ 2c
  const uint32_t koff0 = rowperm(l32) * RB + ((half ^ swz<D>(rowperm(l32))) << 4);
  uint32_t voff[ND][2];  // V rows: key 16 t + 8 half + 4 sub + (lane & 15) / 4
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int key = 8 * half + 4 * sub + ((lane & 15) >> 2);
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db][sub] = SUB_B + key * RB + ((((col >> 3) ^ swz<D>(key)) << 4) | ((col & 7) << 1));
    }
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v ones = {(__bf16)1.0f, (__bf16)1.0f};

  if constexpr (!PIPE) {
    // one sub-tile in buffer tb: S^T = K Q^T (2 blocks of 32 keys), softmax, O^T += V^T P^T;
    // the copies of the next sub-tile (offsets ko, into buffer nb) go out during the S MFMAs
    auto compute = [&](int nvalid, const char* tb, char* nb, const uint32_t (&ko)[NLD]) {
      f32x16 s[2];
      s[0] = f32x16{};
      s[1] = f32x16{};
      bf16x8 a[3][2];
      auto kfrag = [&](int c, int kb) {
        return *reinterpret_cast<const bf16x8*>(tb + (koff0 ^ (uint32_t)(c << 5)) + 32 * kb * RB);
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) a[0][kb] = kfrag(0, kb);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) a[1][kb] = kfrag(1, kb);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 2 < NC) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) a[(c + 2) % 3][kb] = kfrag(c + 2, kb);
        }
        if (c < NLD) copy16_async(kbase, ko[c], nb + row0 * RB + c * 1024);
        else if (c < 2 * NLD) copy16_async(vbase, ko[c - NLD], nb + SUB_B + row0 * RB + (c - NLD) * 1024);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c % 3][kb], qf[c], s[kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the fragments of chunks 0 and 1
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                  // the MFMAs of chunk c
        if (c + 2 < NC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the fragments of chunk c + 2
      }
      // accumulator j of key block kb holds key 32*kb + 16*(j/8) + 8*half + j%8
      if (nvalid < kSub) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * kb + 16 * (j / 8) + 8 * half + (j % 8) >= nvalid) s[kb][j] = -INFINITY;
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
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
      bf16x8 pb[4];  // P^T chunk t holds keys 16t + 8*half + e
      float lsum = l_run;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
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
      auto vfrag = [&](int t, int db) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((UF_LDS i16x4*)(tb + voff[db][0] + 16 * t * RB));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((UF_LDS i16x4*)(tb + voff[db][1] + 16 * t * RB));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 va[2][ND];
#pragma unroll
      for (int db = 0; db < ND; ++db) va[0][db] = vfrag(0, db);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t + 1 < 4) {
#pragma unroll
          for (int db = 0; db < ND; ++db) va[(t + 1) & 1][db] = vfrag(t + 1, db);
        }
#pragma unroll
        for (int db = 0; db < ND; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t & 1][db], pb[t], o[db], 0, 0, 0);
      }
    };

    // ---- main loop over sub-tiles (kept tile kt gives sub-tiles 2 kt and 2 kt + 1; the second is
    // skipped when it holds no visible key).  Sub-tile j sits in buffer j % 2.
    bool own_t = false, own_n = false;
    int kt = tiles.next(lane, own_t);
    int h = 0;
    uint32_t ko[NLD];
    copy_offsets(kt >= 0 ? kt * kAttnTileKeys : -1, ko);
#pragma unroll
    for (int i = 0; i < NLD; ++i) copy16_async(kbase, ko[i], smem + row0 * RB + i * 1024);
#pragma unroll
    for (int i = 0; i < NLD; ++i) copy16_async(vbase, ko[i], smem + SUB_B + row0 * RB + i * 1024);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int j = 0; kt >= 0; ++j) {
      // the next sub-tile
      int nkt = kt, nh = 1;
      own_n = own_t;
      if (h == 1 || kt * kAttnTileKeys + kSub >= p.n_k) {
        nkt = tiles.next(lane, own_n);
        nh = 0;
      }
      copy_offsets(nkt >= 0 ? nkt * kAttnTileKeys + nh * kSub : -1, ko);
      const char* tb = smem + (j & 1) * 2 * SUB_B;
      char* nb = smem + ((j + 1) & 1) * 2 * SUB_B;
      if (own_t) {
        compute(min(kSub, p.n_k - (kt * kAttnTileKeys + h * kSub)), tb, nb, ko);
      } else {
#pragma unroll
        for (int i = 0; i < NLD; ++i) copy16_async(kbase, ko[i], nb + row0 * RB + i * 1024);
#pragma unroll
        for (int i = 0; i < NLD; ++i) copy16_async(vbase, ko[i], nb + SUB_B + row0 * RB + i * 1024);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // sub-tile j + 1 is in LDS and every wave is done with sub-tile j
      kt = nkt;
      h = nh;
      own_t = own_n;
    }
  } else {
    // ---- software-pipelined loop.  Sub-tile j has K in buffer pair j % 2 and V in the same pair.
    // Iteration j multiplies S of sub-tile j + 1 while it exponentiates the scores of sub-tile j,
    // then P.V of sub-tile j, then takes the maximum of the new scores.  K is copied two
    // sub-tiles ahead, V one ahead: during iteration j the copies write K of j + 2 into pair j % 2
    // (its K was last read in iteration j - 1) and V of j + 1 into pair (j + 1) % 2 (its V was last
    // read in iteration j - 1).
    struct Sub { int kt, h; bool own; };
    auto sub_j0 = [&](const Sub& s) { return s.kt >= 0 ? s.kt * kAttnTileKeys + s.h * kSub : -1; };
    auto advance = [&](const Sub& s) {
      Sub n = s;
      if (s.kt < 0) return n;
      if (s.h == 0 && s.kt * kAttnTileKeys + kSub < p.n_k) {
        n.h = 1;
        return n;
      }
      bool own = false;
      n.kt = tiles.next(lane, own);
      n.h = 0;
      n.own = own;
      return n;
    };
    auto kbuf = [&](int j) -> char* { return smem + (j & 1) * 2 * SUB_B; };
    // the scores of the sub-tile whose K sits at kb; copies (K with offsets ck into kd, V with cv
    // into vd) go out one per d chunk
    auto scores = [&](const char* kb, f32x16 (&sc)[2], const uint32_t (&ck)[NLD], char* kd,
                      const uint32_t (&cv)[NLD], char* vd) {
      sc[0] = f32x16{};
      sc[1] = f32x16{};
      bf16x8 a[3][2];
      auto kfrag = [&](int c, int kbk) {
        return *reinterpret_cast<const bf16x8*>(kb + (koff0 ^ (uint32_t)(c << 5)) + 32 * kbk * RB);
      };
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) a[0][kbk] = kfrag(0, kbk);
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) a[1][kbk] = kfrag(1, kbk);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 2 < NC) {
#pragma unroll
          for (int kbk = 0; kbk < 2; ++kbk) a[(c + 2) % 3][kbk] = kfrag(c + 2, kbk);
        }
        if (c < NLD) copy16_async(kbase, ck[c], kd + row0 * RB + c * 1024);
        else if (c < 2 * NLD) copy16_async(vbase, cv[c - NLD], vd + row0 * RB + (c - NLD) * 1024);
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
          sc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c % 3][kbk], qf[c], sc[kbk], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (c + 2 < NC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    };
    // keys past the sub-tile's visible ones, or every key of a sub-tile this wave does not own, score -inf
    auto mask_scores = [&](const Sub& s, f32x16 (&sc)[2]) {
      const int nv = s.kt >= 0 && s.own ? min(kSub, p.n_k - sub_j0(s)) : 0;
      if (nv < kSub) {
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * kbk + 16 * (j / 8) + 8 * half + (j % 8) >= nv) sc[kbk][j] = -INFINITY;
      }
    };
    auto row_max = [&](const f32x16 (&sc)[2]) {
      float mx = sc[0][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[kbk][j]);
      return max_xor32(mx);
    };
    // move the reference point when the running max has grown by more than 2^8 (lazy rescaling)
    auto update_ref = [&](float mx) {
      const float m_new = fmaxf(m_run, mx);
      const bool need = (m_new - m_run) * c2 > 8.f;
      if (__ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c2) : 1.f;
        if (need) m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i) o[i] *= alpha;
      }
    };
    // probabilities of key block kbk (P^T chunks 2 kbk and 2 kbk + 1) against reference mc
    auto probs = [&](const f32x16 (&sc)[2], int kbk, float mc, bf16x8 (&pb)[4], float& lsum) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][8 * hf + e], c2, -mc));
        const bf16x8 pk = __builtin_convertvector(pv, bf16x8);
        pb[2 * kbk + hf] = pk;
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 0, 1), ones, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 2, 3), ones, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 4, 5), ones, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk, pk, 6, 7), ones, lsum, false);
      }
    };
    auto vfrag = [&](const char* tb, int t, int db) {
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((UF_LDS i16x4*)(tb + voff[db][0] + 16 * t * RB));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((UF_LDS i16x4*)(tb + voff[db][1] + 16 * t * RB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // P.V chunks t0 and t0 + 1 (va[t0 & 1] holds chunk t0's fragments; the next chunk's are read ahead)
    auto pv_pair = [&](const char* tb, const bf16x8 (&pb)[4], int t0, bf16x8 (&va)[2][ND]) {
#pragma unroll
      for (int t = t0; t < t0 + 2; ++t) {
        if (t + 1 < 4) {
#pragma unroll
          for (int db = 0; db < ND; ++db) va[(t + 1) & 1][db] = vfrag(tb, t + 1, db);
        }
#pragma unroll
        for (int db = 0; db < ND; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t & 1][db], pb[t], o[db], 0, 0, 0);
      }
    };
    auto pv_mfma = [&](const char* tb, const bf16x8 (&pb)[4]) {
      bf16x8 va[2][ND];
#pragma unroll
      for (int db = 0; db < ND; ++db) va[0][db] = vfrag(tb, 0, db);
      pv_pair(tb, pb, 0, va);
      pv_pair(tb, pb, 2, va);
    };
    // the reference point in log2 units; 0 while this wave has seen no visible key (every score so
    // far -inf), so that the probabilities of an unkept sub-tile come out 0 instead of NaN
    auto ref_of = [&]() { return m_run == -INFINITY ? 0.f : m_run * c2; };

    Sub s0;
    {
      bool own = false;
      s0.kt = tiles.next(lane, own);
      s0.h = 0;
      s0.own = own;
    }
    Sub s1 = advance(s0);
    uint32_t ko0[NLD], ko1[NLD], ko2[NLD];
    copy_offsets(sub_j0(s0), ko0);
    copy_offsets(sub_j0(s1), ko1);
#pragma unroll
    for (int i = 0; i < NLD; ++i) copy16_async(kbase, ko0[i], smem + row0 * RB + i * 1024);
#pragma unroll
    for (int i = 0; i < NLD; ++i) copy16_async(vbase, ko0[i], smem + SUB_B + row0 * RB + i * 1024);
#pragma unroll
    for (int i = 0; i < NLD; ++i) copy16_async(kbase, ko1[i], smem + 2 * SUB_B + row0 * RB + i * 1024);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 sa[2], sb[2];
    if (s0.kt >= 0) {
      // scores of sub-tile 0; the copies that go out with them write K and V of sub-tile 1 into
      // pair 1, which nothing reads before the barrier below (K is the same data again)
      scores(kbuf(0), sa, ko1, kbuf(1), ko1, kbuf(1) + SUB_B);
      mask_scores(s0, sa);
      update_ref(row_max(sa));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with K of sub-tile 0, which iteration 0 overwrites
    // one iteration: cur holds the scores of sub-tile j (s0), nxt receives those of j + 1 (s1)
    auto iteration = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
      const Sub s2 = advance(s1);
      copy_offsets(sub_j0(s2), ko2);
      const float mc = ref_of();
      bf16x8 pb[4];
      float lsum = l_run;
      scores(kbuf(j + 1), nxt, ko2, kbuf(j), ko1, kbuf(j + 1) + SUB_B);
      probs(cur, 0, mc, pb, lsum);
      bf16x8 va[2][ND];
#pragma unroll
      for (int db = 0; db < ND; ++db) va[0][db] = vfrag(kbuf(j), 0, db);
      pv_pair(kbuf(j), pb, 0, va);
      probs(cur, 1, mc, pb, lsum);
      l_run = lsum;
      pv_pair(kbuf(j), pb, 2, va);
      mask_scores(s1, nxt);
      update_ref(row_max(nxt));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      s0 = s1;
      s1 = s2;
#pragma unroll
      for (int i = 0; i < NLD; ++i) ko1[i] = ko2[i];
    };
    int j = 0;
    if (s0.kt >= 0) {
      while (s1.kt >= 0) {
        iteration(j, sa, sb);
        ++j;
        if (s1.kt < 0) break;
        iteration(j, sb, sa);
        ++j;
      }
      // the last sub-tile: its probabilities and P.V
      const f32x16 (&last)[2] = (j & 1) ? sb : sa;
      const float mc = ref_of();
      bf16x8 pb[4];
      float lsum = l_run;
      probs(last, 0, mc, pb, lsum);
      probs(last, 1, mc, pb, lsum);
      l_run = lsum;
      pv_mfma(kbuf(j), pb);
    }
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

}  // namespace
}  // namespace uf
