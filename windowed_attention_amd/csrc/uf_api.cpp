// Host side of libuf: argument validation, the rolling-window bookkeeping
// and launch configuration.  See include/uf.h for the contract of each call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>

#include "uf.h"
#include "uf_internal.h"

static_assert(uf::kStaticScratchBytes == UF_STATIC_SCRATCH_BYTES, "scratch size and its header constant");

struct uf_kvcache {
  uf_kvcache_desc d;
  int64_t frames;       // frames appended since create / reset
  int32_t last_append;  // frames in the newest append
  int32_t active;       // recent frames visible (crop), 1..W
  int32_t block_frames; // block order: frames per step of this stream (0 until the first append)
};

namespace {

thread_local std::string g_last_error;

uf_status fail(uf_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

uf_status hip_fail(hipError_t e, const char* what) {
  return fail(UF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxIndex = (int64_t)1 << 31;
constexpr int kMaxSplits = 16;
constexpr int kPipelineMinTiles = 16;  // key tiles per part from which the pipelined loop is taken

float fp8_attention_q_scale(const uf_kvcache_desc& d, int* e_out);

uf_status check_desc(const uf_kvcache_desc* d) {
  if (!d) return fail(UF_ERR_INVALID_ARG, "desc is NULL");
  if (d->n_kv_heads < 1) return fail(UF_ERR_SHAPE, "n_kv_heads must be >= 1 (got %d)", d->n_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(UF_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->tokens_per_frame < 1) return fail(UF_ERR_SHAPE, "tokens_per_frame must be >= 1");
  if (d->window_frames < 1) return fail(UF_ERR_SHAPE, "window_frames must be >= 1");
  if (d->anchor_frames < 0) return fail(UF_ERR_SHAPE, "anchor_frames must be >= 0");
  // the attention kernels address a head's K or V storage with 32-bit byte offsets
  const int64_t rows = (int64_t)(d->anchor_frames + (int64_t)d->window_frames) * d->tokens_per_frame;
  if (rows >= kMaxIndex || rows * d->head_dim * (d->kv_dtype == UF_FP8_E4M3 ? 1 : 2) >= ((int64_t)1 << 32))
    return fail(UF_ERR_CAPACITY, "cache of %lld rows per head is too large (at most 4 GiB per head and tensor)",
                (long long)rows);
  if ((d->block_grid_h == 0) != (d->block_grid_w == 0) || d->block_grid_h < 0 || d->block_grid_w < 0 ||
      (d->block_grid_h && (int64_t)d->block_grid_h * d->block_grid_w != d->tokens_per_frame))
    return fail(UF_ERR_SHAPE, "block grid %d x %d does not give %d tokens per frame", d->block_grid_h,
                d->block_grid_w, d->tokens_per_frame);
  if (d->max_q_heads < 0 || d->max_q_tokens < 0)
    return fail(UF_ERR_INVALID_ARG, "max_q_heads and max_q_tokens must be >= 0");
  if (d->heads_per_wg != 0 && d->heads_per_wg != 1 && d->heads_per_wg != 2 && d->heads_per_wg != 4)
    return fail(UF_ERR_INVALID_ARG, "heads_per_wg must be 0, 1, 2 or 4 (got %d)", d->heads_per_wg);
  if (d->splits < 0 || d->splits > kMaxSplits)
    return fail(UF_ERR_INVALID_ARG, "splits must lie in 0..%d (got %d)", kMaxSplits, d->splits);
  if (d->pipeline < 0 || d->pipeline > 2)
    return fail(UF_ERR_INVALID_ARG, "pipeline must be 0, 1 or 2 (got %d)", d->pipeline);
  if (d->kv_dtype != UF_BF16 && d->kv_dtype != UF_FP8_E4M3)
    return fail(UF_ERR_DTYPE, "kv_dtype must be UF_BF16 or UF_FP8_E4M3 (got %d)", d->kv_dtype);
  if (d->kv_dtype == UF_FP8_E4M3) {
    const float sc[3] = {d->q_scale, d->k_scale, d->v_scale};
    for (float x : sc)
      if (!(x > 0.f) || !isfinite(x) || !isfinite(1.0f / x))
        return fail(UF_ERR_INVALID_ARG, "FP8 scales must be positive, finite and invertible");
    int e = 0;
    const float qs = fp8_attention_q_scale(*d, &e);
    if (e < -120 || e > 120 || !(qs > 0.f) || !isfinite(qs) || !isfinite(1.0f / qs))
      return fail(UF_ERR_INVALID_ARG, "FP8 scales: log2(e)/sqrt(head_dim) q_scale k_scale = 2^%d is out of range", e);
  }
  return UF_OK;
}

int elem_bytes(const uf_kvcache_desc& d) { return d.kv_dtype == UF_FP8_E4M3 ? 1 : 2; }
float inv_scale(float s) { return (float)(1.0 / (double)s); }

// The scale an FP8 step quantizes q with: q_scale rounded up, by less than a factor of two, so
// that the product of the softmax factor log2(e)/sqrt(d) and the two scales is a power of two
// 2^e (e = ceil(log2(log2(e)/sqrt(d) q_scale k_scale))).  The kernel then applies 2^e as the
// Q operand's E8M0 scale and gets the scores in log2 units with no multiply.  Computed in
// double from the float scales and rounded to float.
float fp8_attention_q_scale(const uf_kvcache_desc& d, int* e_out) {
  const double c0 = 1.4426950408889634 / sqrt((double)d.head_dim);
  const double x = c0 * (double)d.q_scale * (double)d.k_scale;
  int e = 0;
  const double f = frexp(x, &e);  // x = f 2^e, f in [0.5, 1)
  if (f == 0.5) e -= 1;           // x is a power of two already
  *e_out = e;
  return (float)(ldexp(1.0, e) / (c0 * (double)d.k_scale));
}

int64_t rows_per_head(const uf_kvcache_desc& d) {
  return ((int64_t)d.anchor_frames + d.window_frames) * d.tokens_per_frame;
}

// Window after `frames` frames appended with a crop of `active` recent frames.
uf_window_info window_of(const uf_kvcache_desc& d, int64_t frames, int32_t last_append, int32_t active) {
  uf_window_info w;
  memset(&w, 0, sizeof w);
  const int64_t L = d.tokens_per_frame;
  const int64_t anchors = std::min<int64_t>(frames, d.anchor_frames);
  const int64_t recent_total = frames - anchors;
  const int64_t recent = std::min<int64_t>(recent_total, active);
  const int64_t oldest = recent_total - recent;  // recent-frame index of the oldest visible one
  w.frames_appended = frames;
  w.anchor_keys = (int32_t)(anchors * L);
  w.ring_keys = (int32_t)(recent * L);
  w.n_keys = w.anchor_keys + w.ring_keys;
  w.ring_capacity_keys = (int32_t)((int64_t)d.window_frames * L);
  w.ring_rotation_keys = (int32_t)((oldest % d.window_frames) * L);
  w.last_append_frames = last_append;
  w.active_frames = active;
  return w;
}

int64_t first_row_of_frame(const uf_kvcache_desc& d, int64_t frame) {
  const int64_t slot = frame < d.anchor_frames ? frame
                                               : d.anchor_frames + (frame - d.anchor_frames) % d.window_frames;
  return slot * d.tokens_per_frame;
}

uf_status check_append_request(const uf_kvcache* c, int32_t n_frames, uint32_t flags) {
  if (flags & ~(UF_APPEND_OVERWRITE_NEWEST | UF_APPEND_COMMIT_ONLY))
    return fail(UF_ERR_INVALID_ARG, "unknown append flags 0x%x", flags);
  if (n_frames < 0) return fail(UF_ERR_INVALID_ARG, "n_frames must be >= 0");
  if (n_frames > UF_MAX_APPEND_FRAMES)
    return fail(UF_ERR_CAPACITY, "at most %d frames per append (got %d)", UF_MAX_APPEND_FRAMES, n_frames);
  const auto& d = c->d;
  if (flags & UF_APPEND_OVERWRITE_NEWEST) {
    if (n_frames != c->last_append || c->last_append == 0)
      return fail(UF_ERR_STATE, "overwrite must cover the newest append exactly (%d frames, got %d)",
                  c->last_append, n_frames);
    return UF_OK;
  }
  if (d.block_grid_h && n_frames > 0) {
    if (c->block_frames && n_frames != c->block_frames)
      return fail(UF_ERR_STATE, "block order: every append of the stream has %d frames (got %d)", c->block_frames,
                  n_frames);
    if (d.anchor_frames % n_frames || d.window_frames % n_frames)
      return fail(UF_ERR_SHAPE, "block order: %d frames per append must divide anchor (%d) and window (%d) frames",
                  n_frames, d.anchor_frames, d.window_frames);
  }
  const int64_t first = c->frames;
  const int64_t anchor_left = std::max<int64_t>(0, d.anchor_frames - first);
  const int64_t ring_frames = std::max<int64_t>(0, n_frames - anchor_left);
  if (ring_frames > d.window_frames)
    return fail(UF_ERR_CAPACITY, "append of %d frames puts %lld frames in a ring of %d", n_frames,
                (long long)ring_frames, d.window_frames);
  return UF_OK;
}

uf_status check_tensor(const uf_tensor* t, const char* name, int head_dim) {
  if (!t) return fail(UF_ERR_INVALID_ARG, "%s is NULL", name);
  if (t->dtype != UF_BF16) return fail(UF_ERR_DTYPE, "%s: dtype must be UF_BF16", name);
  if (t->n_tokens < 0 || t->n_heads < 1) return fail(UF_ERR_SHAPE, "%s: bad sizes", name);
  if (t->head_dim != head_dim)
    return fail(UF_ERR_SHAPE, "%s: head_dim %d, cache has %d", name, t->head_dim, head_dim);
  if (t->n_tokens > 0 && !t->data) return fail(UF_ERR_INVALID_ARG, "%s: data is NULL", name);
  if (((uintptr_t)t->data & 15) != 0) return fail(UF_ERR_INVALID_ARG, "%s: data not 16-byte aligned", name);
  if (t->stride_token < 0 || t->stride_head < 0 || t->stride_token % 8 || t->stride_head % 8)
    return fail(UF_ERR_INVALID_ARG, "%s: strides must be non-negative multiples of 8 elements", name);
  if (t->n_heads > 1 && t->stride_head < head_dim)
    return fail(UF_ERR_SHAPE, "%s: head stride smaller than head_dim", name);
  return UF_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

size_t tensor_extent_bytes(const uf_tensor& t) {
  if (t.n_tokens == 0) return 0;
  return ((size_t)(t.n_tokens - 1) * t.stride_token + (size_t)(t.n_heads - 1) * t.stride_head + t.head_dim) * 2;
}

int device_cu_count() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached_dev = dev;
    cached_cus = cus;
  }
  return cached_cus;
}

// Split partials are budgeted in (split, query, head) rows.  The library's split rule
// (choose_splits) never makes more than four rounds of resident work-groups (2 per CU) out of
// the split work items, 128 rows each, so it never needs more than 4 * 2 * CUs * 128 rows.
int64_t split_row_budget(const uf_kvcache_desc& d) {
  int64_t rows = 4 * 2 * (int64_t)device_cu_count() * UF_TILE;
  if (d.max_q_heads > 0 && d.max_q_tokens > 0)
    rows = std::min<int64_t>(rows, (int64_t)kMaxSplits * d.max_q_heads * d.max_q_tokens);
  return rows;
}

// Key-range parts for a step of `items` work items over n_kt key tiles, on a chip that holds
// `slots` work-groups at once (two per CU), at least 4 key tiles per part.
// - Fewer items than slots: as many parts as keep the whole grid resident (one more part
//   starts a second round of work-groups, which costs more than the shorter ranges save:
//   decoder 3 parts 62 us, 4 parts 74 us).
// - Between one and two rounds of items of a dense step: the last round runs mostly empty,
//   because items of a dense step take about the same time.  Split into the parts (at most 4,
//   at most 4 rounds) that fill the rounds best, when that fills them at least a tenth better
//   than unsplit: decoder-XL (678 items, 1.32 rounds) 3 parts, 209 us instead of 245.  Under
//   a block mask the items keep different numbers of tiles and do not run in rounds: unsplit
//   (decoder-XL under per-head top-k masks, 14 of 57 tiles kept: 3 parts 89 us, unsplit 71).
// - Two rounds or more: unsplit.  Item times spread enough that the last round is not the
//   problem, and partials cost more than they save (1K 2 parts 1.16 ms instead of 1.05).
int choose_splits(int64_t items, int n_kt, int64_t slots, bool masked) {
  const int most = std::max(1, n_kt / 4);
  if (items < slots) return (int)std::min<int64_t>({std::max<int64_t>(1, slots / items), kMaxSplits, most});
  if (masked || items >= 2 * slots) return 1;
  const auto fill = [&](int s) {
    const int64_t wgs = items * s;
    return (double)wgs / (double)(((wgs + slots - 1) / slots) * slots);
  };
  int best = 1;
  for (int s = 2; s <= std::min(4, most); ++s)
    if (items * s <= 4 * slots && fill(s) > fill(best) + 1e-9) best = s;
  return fill(best) >= fill(1) + 0.1 ? best : 1;
}

// Uneven two-part split of a dense head_dim 128 step with more than half a round but less than
// one round of items (480P: 444 items for 512 slots).  Unsplit, the items all start at once
// and the CUs that got one work-group instead of two idle for the last fifth of the step.
// Instead each item is cut into a body (the first 13/16 of its key tiles) and a tail (the
// rest); the grid holds all bodies before all tails, so the tails start on the free slots and
// then on the slots that free up.  Returns the body's key tiles, or 0 for no such split.
// Measured side by side, attention kernel plus combine: 480P 530 -> 510 us (bf16), 314 -> 294 us
// (FP8); a tail of 1/4 or 1/8 gains less, 3/8 nothing.  Under a block mask the items keep
// different numbers of tiles and do not run in lockstep: unsplit.
int body_tiles(int64_t items, int n_kt, int64_t slots, bool masked, int head_dim) {
  if (masked || head_dim != 128 || n_kt < 8 || 2 * items <= slots || items >= slots) return 0;
  return n_kt - (3 * n_kt + 8) / 16;
}

// The crop of a block-order stream must keep whole steps: every frame slot of a step holds
// tokens of all the step's frames.
uf_status check_block_crop(const uf_kvcache* c) {
  if (c->d.block_grid_h && c->block_frames && c->active % c->block_frames)
    return fail(UF_ERR_SHAPE, "block order: the window crop (%d frames) must be a multiple of the %d frames per step",
                c->active, c->block_frames);
  return UF_OK;
}

// Bytes of the query-tile means in the mask-generation workspace, rounded up
// so that the key-tile means after them start 256-byte aligned.
size_t topk_workspace_split(int64_t q_tiles_times_heads, int head_dim) {
  const size_t b = (size_t)q_tiles_times_heads * head_dim * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

size_t uf_kvcache_storage_bytes(const uf_kvcache_desc* desc) {
  if (!desc || check_desc(desc) != UF_OK) return 0;
  return (size_t)desc->n_kv_heads * rows_per_head(*desc) * desc->head_dim * elem_bytes(*desc);
}

size_t uf_attn_workspace_bytes(const uf_kvcache_desc* desc) {
  if (!desc || check_desc(desc) != UF_OK) return 0;
  return (size_t)split_row_budget(*desc) * (desc->head_dim + 2) * sizeof(float);
}

uf_status uf_kvcache_create(const uf_kvcache_desc* desc, uf_kvcache** out) {
  if (!out) return fail(UF_ERR_INVALID_ARG, "out is NULL");
  uf_status s = check_desc(desc);
  if (s != UF_OK) return s;
  if (!desc->k_storage || !desc->v_storage) return fail(UF_ERR_INVALID_ARG, "k_storage / v_storage is NULL");
  if (((uintptr_t)desc->k_storage & 15) || ((uintptr_t)desc->v_storage & 15))
    return fail(UF_ERR_INVALID_ARG, "cache storage must be 16-byte aligned");
  const size_t bytes = uf_kvcache_storage_bytes(desc);
  if (overlaps(desc->k_storage, bytes, desc->v_storage, bytes))
    return fail(UF_ERR_INVALID_ARG, "k_storage and v_storage overlap");
  if (desc->workspace_bytes && !desc->workspace)
    return fail(UF_ERR_INVALID_ARG, "workspace_bytes > 0 with a NULL workspace");
  if ((uintptr_t)desc->workspace & 255) return fail(UF_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  uf_kvcache* c = new (std::nothrow) uf_kvcache;
  if (!c) return fail(UF_ERR_INVALID_ARG, "out of host memory");
  c->d = *desc;
  c->frames = 0;
  c->last_append = 0;
  c->active = desc->window_frames;
  c->block_frames = 0;
  *out = c;
  return UF_OK;
}

uf_status uf_kvcache_destroy(uf_kvcache* cache) {
  delete cache;
  return UF_OK;
}

uf_status uf_kvcache_reset(uf_kvcache* cache) {
  if (!cache) return fail(UF_ERR_INVALID_ARG, "cache is NULL");
  cache->frames = 0;
  cache->last_append = 0;
  cache->active = cache->d.window_frames;
  cache->block_frames = 0;
  return UF_OK;
}

uf_status uf_kvcache_set_window(uf_kvcache* cache, int32_t active_frames) {
  if (!cache) return fail(UF_ERR_INVALID_ARG, "cache is NULL");
  if (active_frames < 1 || active_frames > cache->d.window_frames)
    return fail(UF_ERR_SHAPE, "active_frames must lie in 1..%d (got %d)", cache->d.window_frames, active_frames);
  const int32_t before = cache->active;
  cache->active = active_frames;
  const uf_status s = check_block_crop(cache);
  if (s != UF_OK) cache->active = before;
  return s;
}

uf_status uf_kvcache_window(const uf_kvcache* cache, uf_window_info* out) {
  if (!cache || !out) return fail(UF_ERR_INVALID_ARG, "cache or out is NULL");
  *out = window_of(cache->d, cache->frames, cache->last_append, cache->active);
  return UF_OK;
}

uf_status uf_kvcache_plan_append(const uf_kvcache* cache, int32_t n_frames, uint32_t flags, uf_append_plan* out) {
  if (!cache || !out) return fail(UF_ERR_INVALID_ARG, "cache or out is NULL");
  uf_status s = check_append_request(cache, n_frames, flags);
  if (s != UF_OK) return s;
  memset(out, 0, sizeof *out);
  out->n_frames = n_frames;
  const bool overwrite = flags & UF_APPEND_OVERWRITE_NEWEST;
  const int64_t first = overwrite ? cache->frames - n_frames : cache->frames;
  for (int f = 0; f < n_frames; ++f) out->first_row[f] = (int32_t)first_row_of_frame(cache->d, first + f);
  if (overwrite || n_frames == 0)
    out->window_after = window_of(cache->d, cache->frames, cache->last_append, cache->active);
  else
    out->window_after = window_of(cache->d, cache->frames + n_frames, n_frames, cache->active);
  return UF_OK;
}

uf_status uf_kvcache_append(uf_kvcache* cache, const uf_tensor* k_new, const uf_tensor* v_new, int32_t n_frames,
                            uint32_t flags, void* stream) {
  if (!cache) return fail(UF_ERR_INVALID_ARG, "cache is NULL");
  uf_status s = check_append_request(cache, n_frames, flags);
  if (s != UF_OK) return s;
  if (n_frames == 0) return UF_OK;
  const auto& d = cache->d;
  const bool overwrite = flags & UF_APPEND_OVERWRITE_NEWEST;
  if (flags & UF_APPEND_COMMIT_ONLY) {
    if (k_new || v_new) return fail(UF_ERR_INVALID_ARG, "UF_APPEND_COMMIT_ONLY takes NULL k_new and v_new");
  } else {
    if ((s = check_tensor(k_new, "k_new", d.head_dim)) != UF_OK) return s;
    if ((s = check_tensor(v_new, "v_new", d.head_dim)) != UF_OK) return s;
    const int64_t n_tok = (int64_t)n_frames * d.tokens_per_frame;
    if (k_new->n_tokens != n_tok || v_new->n_tokens != n_tok)
      return fail(UF_ERR_SHAPE, "k_new / v_new must hold n_frames * tokens_per_frame = %lld tokens",
                  (long long)n_tok);
    if (k_new->n_heads != d.n_kv_heads || v_new->n_heads != d.n_kv_heads)
      return fail(UF_ERR_SHAPE, "k_new / v_new must have %d heads", d.n_kv_heads);
    if (n_tok * (d.head_dim / 8) * d.n_kv_heads >= kMaxIndex)
      return fail(UF_ERR_CAPACITY, "append too large for one launch");
    uf::AppendParams p;
    p.src[0] = (const uint16_t*)k_new->data;
    p.src[1] = (const uint16_t*)v_new->data;
    p.src_stride_tok[0] = k_new->stride_token;
    p.src_stride_tok[1] = v_new->stride_token;
    p.src_stride_head[0] = k_new->stride_head;
    p.src_stride_head[1] = v_new->stride_head;
    p.dst[0] = (uint16_t*)d.k_storage;
    p.dst[1] = (uint16_t*)d.v_storage;
    p.rows_total = rows_per_head(d);
    p.n_tok = (int32_t)n_tok;
    p.n_heads = d.n_kv_heads;
    p.head_dim = d.head_dim;
    p.tokens_per_frame = d.tokens_per_frame;
    p.anchor_frames = d.anchor_frames;
    p.window_frames = d.window_frames;
    p.first_frame = overwrite ? cache->frames - n_frames : cache->frames;
    p.blk_h = d.block_grid_h;
    p.blk_w = d.block_grid_w;
    hipError_t e;
    if (d.kv_dtype == UF_FP8_E4M3) {
      uf::AppendFp8Params f;
      f.a = p;
      f.inv_scale[0] = inv_scale(d.k_scale);
      f.inv_scale[1] = inv_scale(d.v_scale);
      e = uf::launch_append_fp8(f, (hipStream_t)stream);
    } else {
      e = uf::launch_append(p, (hipStream_t)stream);
    }
    if (e != hipSuccess) return hip_fail(e, "append launch");
  }
  if (!overwrite) {
    cache->frames += n_frames;
    cache->last_append = n_frames;
  }
  if (d.block_grid_h) cache->block_frames = n_frames;
  return UF_OK;
}

}  // extern "C"

namespace {

// The attention step with split partials in `ws` (ws_bytes bytes, 256-byte aligned, or NULL
// with 0).  With use_static, ws is ignored: the partials go to the library's own per-device
// scratch, and a forced split count whose partials do not fit it is refused.
uf_status attn_step(const uf_tensor* q, uf_kvcache* cache, const uf_block_mask* mask, uf_tensor* out,
                    void* stream, void* ws, size_t ws_bytes, bool use_static) {
  if (!cache) return fail(UF_ERR_INVALID_ARG, "cache is NULL");
  const auto& d = cache->d;
  uf_status s;
  if ((s = check_tensor(q, "q", d.head_dim)) != UF_OK) return s;
  if ((s = check_tensor(out, "out", d.head_dim)) != UF_OK) return s;
  if (out->n_tokens != q->n_tokens || out->n_heads != q->n_heads)
    return fail(UF_ERR_SHAPE, "out must have q's shape");
  if (q->n_heads % d.n_kv_heads != 0)
    return fail(UF_ERR_SHAPE, "query heads (%d) must be a multiple of KV heads (%d)", q->n_heads, d.n_kv_heads);
  const uf_window_info w = window_of(d, cache->frames, cache->last_append, cache->active);
  if (w.n_keys == 0) return fail(UF_ERR_STATE, "no frame appended yet");
  const int32_t n_q = q->n_tokens, hq = q->n_heads;
  if ((int64_t)n_q * hq >= kMaxIndex) return fail(UF_ERR_CAPACITY, "too many query rows");
  const size_t out_bytes = tensor_extent_bytes(*out);
  const size_t kv_bytes = uf_kvcache_storage_bytes(&d);
  if (overlaps(out->data, out_bytes, q->data, tensor_extent_bytes(*q)) ||
      overlaps(out->data, out_bytes, d.k_storage, kv_bytes) || overlaps(out->data, out_bytes, d.v_storage, kv_bytes))
    return fail(UF_ERR_INVALID_ARG, "out overlaps q or the cache");
  if (d.block_grid_h && n_q != 0 && (int64_t)n_q != (int64_t)cache->block_frames * d.tokens_per_frame)
    return fail(UF_ERR_SHAPE, "block order: the queries must be the step's %lld tokens (got %d)",
                (long long)cache->block_frames * d.tokens_per_frame, n_q);
  if ((s = check_block_crop(cache)) != UF_OK) return s;
  const int n_qt = (n_q + UF_TILE - 1) / UF_TILE;
  const int n_kt = (w.n_keys + UF_TILE - 1) / UF_TILE;
  if (mask) {
    if (!mask->data) return fail(UF_ERR_INVALID_ARG, "mask data is NULL");
    if (mask->n_heads != 1 && mask->n_heads != hq)
      return fail(UF_ERR_SHAPE, "mask n_heads must be 1 or %d (got %d)", hq, mask->n_heads);
    if (mask->n_q_blocks != n_qt || mask->n_k_blocks != n_kt)
      return fail(UF_ERR_SHAPE, "mask must be %d x %d tiles for this step (got %d x %d)", n_qt, n_kt,
                  mask->n_q_blocks, mask->n_k_blocks);
    if (mask->stride_head < 0 || mask->stride_qblock < 0)
      return fail(UF_ERR_INVALID_ARG, "mask strides must be non-negative");
  }
  if (n_q == 0) return UF_OK;

  const int group = hq / d.n_kv_heads;
  const bool per_head_mask = mask && mask->n_heads > 1;
  // Query heads of one KV group per work-group.  With a dense or shared mask every head of the
  // work-group keeps the same tiles, so sharing each staged tile is free.  With per-head masks
  // the work-group walks the union of its heads' rows and a wave skips the tiles its own head
  // does not keep; that pays only when the heads' rows overlap, so it is taken on request.
  int hpw = 1;
  if (d.heads_per_wg) {
    hpw = d.heads_per_wg;
    if (group % hpw)
      return fail(UF_ERR_SHAPE, "heads_per_wg %d does not divide the %d query heads per KV head", hpw, group);
  } else if (!per_head_mask) {
    hpw = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  }
  const int qpw = UF_TILE / hpw;
  const int n_qblk = (n_q + qpw - 1) / qpw;
  const int n_hgrp = hq / hpw;
  const int64_t items = (int64_t)n_qblk * n_hgrp;

  const int64_t slots = 2 * (int64_t)device_cu_count();
  int splits = choose_splits(items, n_kt, slots, mask != nullptr);
  int split_tile = 0;
  if (d.splits) {
    splits = std::min(d.splits, n_kt);
  } else if (splits == 1) {
    split_tile = body_tiles(items, n_kt, slots, mask != nullptr, d.head_dim);
    if (split_tile) splits = 2;
  }
  const int64_t rows = (int64_t)n_q * hq;
  if (use_static) ws_bytes = uf::kStaticScratchBytes;
  const auto fits = [&](int s) {
    return s == 1 || (int64_t)s * rows * (d.head_dim + 2) * (int64_t)sizeof(float) <= (int64_t)ws_bytes;
  };
  if (use_static && d.splits && !fits(splits))
    return fail(UF_ERR_CAPACITY, "%d splits of %lld (query, head) rows need %lld bytes of scratch; the library holds %zu",
                splits, (long long)rows, (long long)splits * rows * (d.head_dim + 2) * (long long)sizeof(float),
                uf::kStaticScratchBytes);
  while (splits > 1 && !fits(splits)) --splits;
  if (splits != 2) split_tile = 0;
  if (items * splits >= kMaxIndex) return fail(UF_ERR_CAPACITY, "grid too large");
  if (use_static && splits > 1) {
    hipError_t e = uf::static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
  }

  uf::AttnParams p;
  p.q = (const uint16_t*)q->data;
  p.q_stride_tok = q->stride_token;
  p.q_stride_head = q->stride_head;
  p.out = (uint16_t*)out->data;
  p.o_stride_tok = out->stride_token;
  p.o_stride_head = out->stride_head;
  p.k = (const uint16_t*)d.k_storage;
  p.v = (const uint16_t*)d.v_storage;
  p.kv_head_stride = rows_per_head(d) * d.head_dim;
  p.n_q = n_q;
  p.n_k = w.n_keys;
  p.n_q_heads = hq;
  p.group = group;
  p.heads_per_wg = hpw;
  p.n_qblk = n_qblk;
  p.n_hgrp = n_hgrp;
  p.splits = splits;
  p.split_tile = split_tile;
  p.anchor_keys = w.anchor_keys;
  p.ring_base = d.anchor_frames * d.tokens_per_frame;
  p.ring_cap = w.ring_capacity_keys;
  p.ring_rot = w.ring_rotation_keys;
  p.mask = mask ? mask->data : nullptr;
  p.mask_heads = mask ? mask->n_heads : 1;
  p.n_kb = n_kt;
  p.mask_stride_head = mask ? mask->stride_head : 0;
  p.mask_stride_q = mask ? mask->stride_qblock : 0;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d.head_dim));
  p.ws_o = splits > 1 ? (float*)ws : nullptr;
  p.ws_ml = splits > 1 ? (float*)ws + (size_t)splits * rows * d.head_dim : nullptr;
  p.blk_h = d.block_grid_h;
  p.blk_w = d.block_grid_w;
  p.blk_frames = cache->block_frames;
  // The software-pipelined loop gains on long key walks (1.3-1.5% at the 480P, 1K and 2K
  // steps) and loses on short ones (its first and last sub-tiles run without overlap: the
  // decoder's 8-tile parts are 1.2-1.6% slower), so it is taken when every part spans at least
  // 16 key tiles.  A union walk (per-head masks shared by a work-group's heads) keeps the
  // one-sub-tile loop, which skips the tiles a wave's head does not keep instead of computing
  // them at -inf.
  const int part_tiles = split_tile ? std::min(split_tile, n_kt - split_tile) : n_kt / splits;
  const bool union_walk = per_head_mask && hpw > 1;
  p.pipelined = d.kv_dtype == UF_BF16 && d.head_dim == 128 &&
                (d.pipeline == 2 || (d.pipeline == 0 && part_tiles >= kPipelineMinTiles && !union_walk));
  hipError_t e;
  if (d.kv_dtype == UF_FP8_E4M3) {
    uf::AttnFp8Params f;
    f.a = p;
    int q_exp = 0;
    f.q_inv_scale = inv_scale(fp8_attention_q_scale(d, &q_exp));
    f.q_e8m0 = 127 + q_exp;
    f.v_scale = d.v_scale;
    e = uf::launch_attention_fp8(f, d.head_dim, (hipStream_t)stream);
  } else {
    e = uf::launch_attention(p, d.head_dim, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (splits > 1) {
    uf::CombineParams c;
    c.ws_o = p.ws_o;
    c.ws_ml = p.ws_ml;
    c.out = p.out;
    c.o_stride_tok = p.o_stride_tok;
    c.o_stride_head = p.o_stride_head;
    c.n_q = n_q;
    c.n_q_heads = hq;
    c.splits = splits;
    e = uf::launch_combine(c, d.head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return UF_OK;
}

}  // namespace

extern "C" {

uf_status uf_attn_step(const uf_tensor* q, uf_kvcache* cache, const uf_block_mask* mask, uf_tensor* out,
                       void* stream) {
  if (!cache) return fail(UF_ERR_INVALID_ARG, "cache is NULL");
  return attn_step(q, cache, mask, out, stream, cache->d.workspace, cache->d.workspace_bytes, false);
}

uf_status uf_attn_step_static(const uf_tensor* q, uf_kvcache* cache, const uf_block_mask* mask, uf_tensor* out,
                              void* stream) {
  return attn_step(q, cache, mask, out, stream, nullptr, 0, true);
}

size_t uf_block_mask_workspace_bytes(const uf_kvcache_desc* desc, int32_t n_q_tokens, int32_t n_q_heads) {
  if (!desc || check_desc(desc) != UF_OK || n_q_tokens < 0 || n_q_heads < 1 || n_q_heads % desc->n_kv_heads)
    return 0;
  const int64_t n_qb = ((int64_t)n_q_tokens + UF_TILE - 1) / UF_TILE;
  const int64_t n_kb = (rows_per_head(*desc) + UF_TILE - 1) / UF_TILE;
  return topk_workspace_split(n_qb * n_q_heads, desc->head_dim) +
         (size_t)n_kb * desc->n_kv_heads * desc->head_dim * sizeof(float);
}

uf_status uf_block_mask_topk(const uf_tensor* q, const uf_kvcache* cache, const uf_topk_params* params,
                             uint8_t* mask, float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache) return fail(UF_ERR_INVALID_ARG, "cache is NULL");
  if (!params) return fail(UF_ERR_INVALID_ARG, "params is NULL");
  const auto& d = cache->d;
  uf_status s;
  if ((s = check_tensor(q, "q", d.head_dim)) != UF_OK) return s;
  if (q->n_heads % d.n_kv_heads != 0)
    return fail(UF_ERR_SHAPE, "query heads (%d) must be a multiple of KV heads (%d)", q->n_heads, d.n_kv_heads);
  if (params->top_k < 0 || params->local_blocks < 0)
    return fail(UF_ERR_INVALID_ARG, "top_k and local_blocks must be >= 0");
  const uf_window_info w = window_of(d, cache->frames, cache->last_append, cache->active);
  if (w.n_keys == 0) return fail(UF_ERR_STATE, "no frame appended yet");
  const int32_t n_q = q->n_tokens, hq = q->n_heads;
  if (n_q > w.n_keys)
    return fail(UF_ERR_SHAPE, "%d queries but only %d visible keys: queries must be the newest keys", n_q, w.n_keys);
  if ((s = check_block_crop(cache)) != UF_OK) return s;
  if (d.block_grid_h && n_q != 0 && (int64_t)n_q != (int64_t)cache->block_frames * d.tokens_per_frame)
    return fail(UF_ERR_SHAPE, "block order: the queries must be the step's %lld tokens (got %d)",
                (long long)cache->block_frames * d.tokens_per_frame, n_q);
  const int n_qb = (n_q + UF_TILE - 1) / UF_TILE;
  const int n_kb = (w.n_keys + UF_TILE - 1) / UF_TILE;
  if (n_kb > uf::kTopkMaxKeyTiles)
    return fail(UF_ERR_UNSUPPORTED, "%d key tiles; mask generation handles at most %d", n_kb, uf::kTopkMaxKeyTiles);
  if ((int64_t)n_qb * hq * n_kb >= kMaxIndex) return fail(UF_ERR_CAPACITY, "mask too large");
  if (n_q == 0) return UF_OK;
  if (!mask) return fail(UF_ERR_INVALID_ARG, "mask is NULL");
  const size_t q_part = topk_workspace_split((int64_t)n_qb * hq, d.head_dim);
  const size_t need = q_part + (size_t)n_kb * d.n_kv_heads * d.head_dim * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(UF_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : 0);
  if ((uintptr_t)workspace & 255) return fail(UF_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t mask_bytes = (size_t)hq * n_qb * n_kb;
  if (overlaps(mask, mask_bytes, workspace, need) || (scores && overlaps(scores, 4 * mask_bytes, workspace, need)) ||
      (scores && overlaps(scores, 4 * mask_bytes, mask, mask_bytes)))
    return fail(UF_ERR_INVALID_ARG, "mask, scores and workspace must not overlap");
  if (((uintptr_t)scores & 3) != 0) return fail(UF_ERR_INVALID_ARG, "scores must be 4-byte aligned");

  uf::TopkParams p;
  p.q = (const uint16_t*)q->data;
  p.q_stride_tok = q->stride_token;
  p.q_stride_head = q->stride_head;
  p.k = (const uint16_t*)d.k_storage;
  p.kv_head_stride = rows_per_head(d) * d.head_dim;
  p.k_fp8 = d.kv_dtype == UF_FP8_E4M3;
  p.k_scale = d.k_scale;
  p.n_q = n_q;
  p.n_k = w.n_keys;
  p.n_q_heads = hq;
  p.n_kv_heads = d.n_kv_heads;
  p.anchor_keys = w.anchor_keys;
  p.ring_base = d.anchor_frames * d.tokens_per_frame;
  p.ring_cap = w.ring_capacity_keys;
  p.ring_rot = w.ring_rotation_keys;
  p.n_qb = n_qb;
  p.n_kb = n_kb;
  p.top_k = std::min(params->top_k, n_kb);
  p.local_blocks = std::min(params->local_blocks, n_kb);
  p.qbar = (float*)workspace;
  p.kbar = (float*)((char*)workspace + q_part);
  p.mask = mask;
  p.scores = scores;
  p.blk_h = d.block_grid_h;
  p.blk_w = d.block_grid_w;
  p.blk_frames = cache->block_frames;
  hipError_t e = uf::launch_block_mask_topk(p, d.head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mask generation launch");
  return UF_OK;
}

const char* uf_status_string(uf_status status) {
  switch (status) {
    case UF_OK: return "UF_OK";
    case UF_ERR_INVALID_ARG: return "UF_ERR_INVALID_ARG";
    case UF_ERR_SHAPE: return "UF_ERR_SHAPE";
    case UF_ERR_DTYPE: return "UF_ERR_DTYPE";
    case UF_ERR_CAPACITY: return "UF_ERR_CAPACITY";
    case UF_ERR_STATE: return "UF_ERR_STATE";
    case UF_ERR_HIP: return "UF_ERR_HIP";
    case UF_ERR_UNSUPPORTED: return "UF_ERR_UNSUPPORTED";
  }
  return "UF_ERR_UNKNOWN";
}

const char* uf_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
