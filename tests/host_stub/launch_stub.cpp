// Host-only stand-ins for the kernel launchers of libuf, for building the C ABI's host side
// (uf_api.cpp) without GPU code, e.g. under AddressSanitizer and UndefinedBehaviorSanitizer.
// Each launcher checks the invariants the real kernels rely on for their parameters, counts
// the call and launches nothing.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "uf_internal.h"

namespace {
int g_launches = 0;
int g_last_splits = 0, g_last_split_tile = 0, g_last_pipelined = -1;

void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launch stub: broken launch invariant: %s\n", what);
    abort();
  }
}
}  // namespace

extern "C" int uf_stub_launch_count(void) { return g_launches; }
// key-range parts and body tiles of the last attention launch
extern "C" int uf_stub_last_splits(void) { return g_last_splits; }
extern "C" int uf_stub_last_split_tile(void) { return g_last_split_tile; }
// loop of the last bf16 attention launch (1 = software-pipelined)
extern "C" int uf_stub_last_pipelined(void) { return g_last_pipelined; }

namespace uf {

// stands in for the device array's address: never dereferenced by the stubs
hipError_t static_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>((uintptr_t)1 << 44);
  return hipSuccess;
}

hipError_t launch_append(const AppendParams& p, hipStream_t) {
  require(p.n_tok > 0 && p.n_heads > 0 && (p.head_dim == 64 || p.head_dim == 128), "append sizes");
  require(p.first_frame >= 0 && p.n_tok % p.tokens_per_frame == 0, "append frames");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_append_fp8(const AppendFp8Params& p, hipStream_t s) { return launch_append(p.a, s); }

static void check_attn(const AttnParams& p) {
  require(p.n_q > 0 && p.n_k > 0 && p.n_q_heads > 0 && p.group > 0, "attention sizes");
  require(p.heads_per_wg == 1 || p.heads_per_wg == 2 || p.heads_per_wg == 4, "heads per work-group");
  require(p.group % p.heads_per_wg == 0 && p.n_q_heads % p.heads_per_wg == 0, "heads per work-group divide");
  require(p.splits >= 1 && p.splits <= 16, "splits");
  require(p.splits == 1 || (p.ws_o && p.ws_ml), "split workspace");
  require(p.n_qblk == (p.n_q + 128 / p.heads_per_wg - 1) / (128 / p.heads_per_wg), "query blocks");
  require(p.anchor_keys >= 0 && p.anchor_keys <= p.n_k && p.ring_rot >= 0 && p.ring_rot < p.ring_cap, "window");
  require(p.n_k - p.anchor_keys <= p.ring_cap, "ring keys");
  require(p.split_tile == 0 || (p.splits == 2 && p.split_tile > 0 && p.split_tile < p.n_kb), "uneven split");
  g_last_splits = p.splits;
  g_last_split_tile = p.split_tile;
}

hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t) {
  check_attn(p);
  require(p.pipelined == 0 || (p.pipelined == 1 && head_dim == 128), "attention loop");
  g_last_pipelined = p.pipelined;
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attention_fp8(const AttnFp8Params& p, int, hipStream_t) {
  check_attn(p.a);
  require(p.q_e8m0 >= 7 && p.q_e8m0 <= 247 && p.q_inv_scale > 0.f && p.v_scale > 0.f, "fp8 attention scales");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_combine(const CombineParams& p, int, hipStream_t) {
  require(p.splits > 1 && p.n_q > 0 && p.ws_o && p.ws_ml, "combine");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_block_mask_topk(const TopkParams& p, int, hipStream_t) {
  require(p.n_qb > 0 && p.n_kb > 0 && p.n_kb <= kTopkMaxKeyTiles && p.qbar && p.kbar && p.mask, "top-k");
  ++g_launches;
  return hipSuccess;
}

}  // namespace uf
