/*
 * uf.h -- C ABI of libuf: chunk-causal attention over a bounded rolling KV
 * cache on one AMD Instinct MI355X (gfx950).
 *
 * What it computes.  A stream is processed in steps.  Each step appends the
 * keys and values of some whole latent frames to a cache, then lets queries
 * attend to the keys the cache currently exposes:
 *
 *   out[i, h, :] = sum_j softmax_j( q[i,h,:] . k[j,g,:] / sqrt(d) ) v[j,g,:]
 *
 * over the visible keys j, with g = floor(h * Hkv / Hq) (grouped-query
 * attention, consecutive query heads sharing a KV head).
 *   - FlashDecoder review, "Rolling KV cache" and Eq. 4: the cache keeps a
 *     fixed window of W frames (the current frames included) per KV group,
 *     so memory and latency do not grow with the video length.
 *   - FlashDecoder review, Algorithm 1: the update keeps the newest frames
 *     and appends the new frame's K/V after them; keys are ordered oldest
 *     to newest.
 *   - FlashDecoder review, "causality by processing order": no mask inside
 *     the window; queries see every visible key, their own frames included.
 *   - HiStream summary, innovation 2 (anchor-guided sliding window): the
 *     first A frames appended stay pinned as an anchor ahead of the window.
 *   - Ultra Flash notes, key design 3 (dynamic block-sparse causal
 *     attention): an optional mask over 128-token blocks says which
 *     (query tile, key tile) pairs are computed at all.
 *   - Ultra Flash notes, key design 4 (dynamic cache management, item iii):
 *     the recent window can be cropped at run time.
 *
 * Conventions for every call.
 *   - Device memory is owned by the caller: cache storage, workspace, q,
 *     k/v inputs, outputs and masks.  The library owns only the host-side
 *     handle.  It never allocates or frees device memory, never
 *     synchronises, never reads device memory on the host, and launches
 *     only on the stream it is given (NULL = the null stream).
 *   - Calls that take a stream return once their kernels are queued.  The
 *     caller orders appends and steps on one stream (or with events).
 *   - Arguments are validated on the host before anything is launched.  On
 *     any error nothing is launched, the cache state is unchanged, a
 *     negative uf_status is returned and uf_last_error() describes it.
 *   - Handles are not thread-safe; distinct handles may be used from
 *     distinct threads.  No C++ exception crosses this interface.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 */
#ifndef UF_H
#define UF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum uf_status {
  UF_OK = 0,
  UF_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad flag, misaligned pointer */
  UF_ERR_SHAPE = -2,        /* sizes disagree with each other or with the cache */
  UF_ERR_DTYPE = -3,        /* element type other than UF_BF16 */
  UF_ERR_CAPACITY = -4,     /* more frames than the ring holds, or index ranges beyond 2^31 */
  UF_ERR_STATE = -5,        /* call not valid in the cache's current state */
  UF_ERR_HIP = -6,          /* the HIP runtime reported an error (message in uf_last_error) */
  UF_ERR_UNSUPPORTED = -7   /* valid request the library does not implement (e.g. head_dim) */
} uf_status;

typedef enum uf_dtype {
  UF_BF16 = 0,     /* bfloat16 */
  UF_FP8_E4M3 = 1  /* OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits, max 448 */
} uf_dtype;

/* Flags of uf_kvcache_append. */
#define UF_APPEND_OVERWRITE_NEWEST 1u /* rewrite the newest append's frames in place; counter unchanged */
#define UF_APPEND_COMMIT_ONLY 2u      /* the caller already wrote the frames at the rows that
                                         uf_kvcache_plan_append reports: advance the counter, copy nothing */

#define UF_TILE 128            /* block-mask tile, in tokens */
#define UF_MAX_APPEND_FRAMES 64 /* frames per uf_kvcache_append call */

typedef struct uf_kvcache uf_kvcache; /* opaque host handle */

/*
 * A device tensor of bf16 in token-major layout [n_tokens, n_heads, head_dim]
 * (the layout a token-wise projection produces, FlashDecoder review, Eq. 3).
 * Element (t, h, c) is at data + t*stride_token + h*stride_head + c; strides
 * are in elements.  The head_dim axis is contiguous.  data must be 16-byte
 * aligned and both strides multiples of 8 elements.
 */
typedef struct uf_tensor {
  void* data;
  int32_t dtype;     /* uf_dtype */
  int32_t n_tokens;
  int32_t n_heads;
  int32_t head_dim;
  int64_t stride_token;
  int64_t stride_head;
} uf_tensor;

/*
 * Cache description.  Storage for K and for V is caller-allocated device
 * memory of uf_kvcache_storage_bytes(desc) bytes each, laid out head-major
 * [n_kv_heads][(anchor_frames + window_frames) * tokens_per_frame][head_dim]
 * elements of kv_dtype (FlashDecoder review, Eq. 4: K_t, V_t in
 * R^{G x (W L) x D_h}).  Rows
 * [0, A*L) hold the anchor frames in append order; rows [A*L, (A+W)*L) are
 * the ring, frame r (counting non-anchor frames from 0) in slot r mod W.
 * The workspace (optional, may be NULL with workspace_bytes 0) holds
 * split-KV partial results; uf_attn_workspace_bytes gives the size that
 * lets the library split whenever it wants to.  Must be 256-byte aligned.
 *
 * kv_dtype selects the storage element type.  UF_BF16 (0) stores the values
 * appended.  UF_FP8_E4M3 stores one byte per element with static scales
 * (FlashDecoder review, inference optimisations: statically calibrated FP8):
 * k and v are stored as E4M3(x / k_scale) and E4M3(x / v_scale), and every
 * step quantizes its queries as E4M3(q / q_scale'), where q_scale' is q_scale
 * rounded up, by less than a factor of two, so that
 * log2(e)/sqrt(head_dim) * q_scale' * k_scale is a power of two 2^e (computed in
 * double from the float scales: e = ceil(log2 of that product with q_scale),
 * q_scale' = float(2^e / (log2(e)/sqrt(head_dim) * k_scale)); e must lie in
 * -120..120); E4M3() rounds to nearest
 * (ties to even; the quotient is x times the reciprocal of the float scale,
 * computed in double and rounded to float, the product rounded to float) and
 * saturates at +-448; a value that rounds to zero keeps its sign.  The step then attends over the dequantized
 * values; its probabilities are rounded to E4M3 for the P.V product.  The
 * scales are ignored for UF_BF16 and must be positive and finite for FP8.
 *
 * Block order (Ultra Flash notes, key design 3: the block-sparse mask is over
 * (2,8,8) spatio-temporal blocks).  With block_grid_h/w set, every append of
 * F frames (F the same for the whole stream, dividing anchor_frames and
 * window_frames) stores the step's tokens, given in raster order (frame, row,
 * column), in block order: the frame pairs' full (2,8,8) blocks, pair by pair,
 * blocks row-major, inside a block frame, row, column; then the odd last
 * frame's full 8x8 patches; then every remaining token (rows from
 * 8*floor(H/8) on, or columns from 8*floor(W/8) on) in raster order.  Key
 * order and 128-token key tiles follow that order.  A step's queries must be
 * the step's F*L tokens, given and returned in raster order; query row i
 * (the unit of query tiles and mask rows) is the token at block position i.
 * The attention output does not depend on the order: it only changes which
 * tokens share a tile.
 */
typedef struct uf_kvcache_desc {
  int32_t n_kv_heads;       /* G >= 1 */
  int32_t head_dim;         /* 64 or 128 */
  int32_t tokens_per_frame; /* L = H' * W' >= 1 */
  int32_t window_frames;    /* W >= 1: recent frames visible, the newest append included */
  int32_t anchor_frames;    /* A >= 0: first frames appended, pinned for the whole stream */
  void* k_storage;
  void* v_storage;
  void* workspace;
  size_t workspace_bytes;
  int32_t kv_dtype;         /* uf_dtype of the storage: UF_BF16 (0) or UF_FP8_E4M3 */
  float q_scale;            /* FP8 static scales (see above) */
  float k_scale;
  float v_scale;
  int32_t block_grid_h;     /* 0, or the frame's token grid (block_grid_h * block_grid_w = L): */
  int32_t block_grid_w;     /* each step is held in (2,8,8) block order (see below) */
  int32_t max_q_heads;      /* 0, or the most query heads a step will have */
  int32_t max_q_tokens;     /* 0, or the most queries a step will have; with max_q_heads it caps
                               uf_attn_workspace_bytes (see there) */
  int32_t heads_per_wg;     /* 0 = the library's choice; 1, 2 or 4: query heads of one KV group
                               that share each staged key tile (must divide Hq / n_kv_heads) */
  int32_t splits;           /* 0 = the library's choice; 1..16: parts of the key range computed
                               apart and merged (fewer when the workspace or the key tiles do not
                               allow as many) */
  int32_t pipeline;         /* attention loop of a bf16 cache at head_dim 128: 0 = the library's
                               choice (software-pipelined when every part of the key range spans
                               at least 16 key tiles and the work-group's heads do not walk the
                               union of per-head mask rows), 1 = one 64-key sub-tile per step,
                               2 = software-pipelined (the scores of the next sub-tile are
                               multiplied while the current one's probabilities are computed).
                               Both give the same results bit for bit; other caches ignore it */
} uf_kvcache_desc;

/*
 * Block mask over 128x128-token tiles, uint8 in device memory, 0 = skip,
 * nonzero = keep (Ultra Flash notes, key design 3: per-head kept blocks).
 * Element (h, qb, kb) is at data + h*stride_head + qb*stride_qblock + kb.
 * n_heads is 1 (one mask shared by all query heads) or the query head
 * count.  n_q_blocks must equal ceil(Nq / 128) and n_k_blocks
 * ceil(n_keys / 128) for the step, tiles taken in query order and in key
 * order (anchor keys, then the recent frames oldest to newest).  A query
 * whose row keeps no tile outputs zeros.
 */
typedef struct uf_block_mask {
  const uint8_t* data;
  int32_t n_heads;
  int32_t n_q_blocks;
  int32_t n_k_blocks;
  int64_t stride_head;
  int64_t stride_qblock;
} uf_block_mask;

/*
 * The keys a step would see now, in key order: anchor_keys anchor rows,
 * then ring_keys recent rows.  Recent key i (0-based) lives in storage row
 * anchor_frames*L + ((i + ring_rotation_keys) mod ring_capacity_keys).
 */
typedef struct uf_window_info {
  int64_t frames_appended;
  int32_t n_keys;
  int32_t anchor_keys;
  int32_t ring_keys;
  int32_t ring_capacity_keys;   /* window_frames * tokens_per_frame */
  int32_t ring_rotation_keys;
  int32_t last_append_frames;
  int32_t active_frames;        /* the crop set by uf_kvcache_set_window (default window_frames) */
} uf_window_info;

/* Where the frames of the next append would go (uf_kvcache_plan_append). */
typedef struct uf_append_plan {
  int32_t n_frames;
  int32_t first_row[UF_MAX_APPEND_FRAMES]; /* storage row of each frame's first token */
  uf_window_info window_after;
} uf_append_plan;

/* Bytes of K storage (same for V) for this description; 0 if it is invalid. */
size_t uf_kvcache_storage_bytes(const uf_kvcache_desc* desc);

/* Workspace bytes that let every step split its key range as the library
 * would choose: (head_dim + 2) * 4 bytes per (split, query, head) row, for
 * at most 1024 rows per compute unit of the current device (the library
 * splits only steps with fewer than two rounds of work-groups, into at most
 * four rounds, so this never limits its own choice), and at most
 * 16 * max_q_heads * max_q_tokens rows when both are given.  A smaller
 * workspace means fewer splits; a forced split count (desc splits) that
 * would need more is lowered to what fits.  0 if invalid. */
size_t uf_attn_workspace_bytes(const uf_kvcache_desc* desc);

/* Validate desc and create a handle with no frames appended.  The storage
 * contents are not touched.  *out is set only on UF_OK.  UF_ERR_CAPACITY when
 * one head's K (or V) storage, (anchor_frames + window_frames) x tokens_per_frame
 * rows of head_dim elements, reaches 4 GiB: the kernels address it with 32-bit
 * byte offsets. */
uf_status uf_kvcache_create(const uf_kvcache_desc* desc, uf_kvcache** out);

/* Free the handle (NULL is accepted).  The caller frees the device memory. */
uf_status uf_kvcache_destroy(uf_kvcache* cache);

/* Start a new stream: frame counter and crop back to their initial values.
 * Storage is left as it is; a later step only reads rows appended since. */
uf_status uf_kvcache_reset(uf_kvcache* cache);

/* Crop the recent window to its newest active_frames frames, 1..window_frames
 * (Ultra Flash notes, key design 4, item iii).  Takes effect at the next step.
 * In block order a step's frames share their tiles, so the crop must be a
 * multiple of the stream's frames per append: UF_ERR_SHAPE here once that
 * count is known, and from uf_attn_step / uf_block_mask_topk otherwise. */
uf_status uf_kvcache_set_window(uf_kvcache* cache, int32_t active_frames);

/*
 * Append n_frames whole frames of keys and values (FlashDecoder review,
 * Algorithm 1, cache update).  k_new and v_new are [n_frames*L, n_kv_heads,
 * head_dim] bf16.  The first anchor_frames frames ever appended go to the
 * anchor rows; later frames go to ring slot (r mod W).  At most W ring frames
 * per call and UF_MAX_APPEND_FRAMES in all.  n_frames == 0 is a no-op.
 * flags: 0, UF_APPEND_OVERWRITE_NEWEST (n_frames must equal the last
 * append's count; the same rows are rewritten, the counter does not move),
 * or UF_APPEND_COMMIT_ONLY (k_new and v_new must be NULL; nothing is copied).
 * One kernel launch on `stream` (none for COMMIT_ONLY); the host frame
 * counter advances when the call returns UF_OK.
 */
uf_status uf_kvcache_append(uf_kvcache* cache, const uf_tensor* k_new, const uf_tensor* v_new,
                            int32_t n_frames, uint32_t flags, void* stream);

/* Host-only: the storage rows the next append of n_frames frames with these
 * flags would write, and the window it would leave.  Changes nothing. */
uf_status uf_kvcache_plan_append(const uf_kvcache* cache, int32_t n_frames, uint32_t flags,
                                 uf_append_plan* out);

/* Host-only: the window a step would see now. */
uf_status uf_kvcache_window(const uf_kvcache* cache, uf_window_info* out);

/*
 * One attention step: every query row of q attends to the cache's visible
 * keys (optionally restricted by block_mask, NULL = all keys).  q and out
 * are [Nq, Hq, head_dim] bf16 with Hq a multiple of n_kv_heads; out must not
 * overlap q or the cache.  Nq == 0 is a no-op.  Accumulation is fp32: scores
 * and the online softmax in fp32, probabilities rounded to bf16 for the
 * P.V product, output rounded to bf16 (nearest even).  UF_ERR_STATE if no
 * frame has been appended.  One or two kernel launches on `stream`.
 */
uf_status uf_attn_step(const uf_tensor* q, uf_kvcache* cache, const uf_block_mask* block_mask,
                       uf_tensor* out, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): uf_attn_step with the same arguments, results and
 * errors, except that split partials go to scratch memory the library holds itself (a
 * file-scope device array of UF_STATIC_SCRATCH_BYTES on each GPU it runs on, kept until the
 * process ends) instead of the cache's workspace, which may then be absent.  Neither this
 * call nor its first use on a device allocates (no hipMalloc, no allocating library routine);
 * its first call on a device looks up the array's device address once.  The split count is
 * chosen as uf_attn_step chooses it with a workspace of UF_STATIC_SCRATCH_BYTES; a split
 * count forced through the cache description (desc splits) whose partials,
 * splits * Nq * Hq * (head_dim + 2) * 4 bytes, exceed UF_STATIC_SCRATCH_BYTES is refused
 * with UF_ERR_CAPACITY.  Every partial is written before it is read, so nothing needs
 * clearing between calls.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (other streams, other threads, other caches) race and must be
 * ordered by the caller.
 */
#define UF_STATIC_SCRATCH_BYTES (32u << 20)
uf_status uf_attn_step_static(const uf_tensor* q, uf_kvcache* cache, const uf_block_mask* block_mask,
                              uf_tensor* out, void* stream);

/*
 * Block-mask generation (Ultra Flash notes, key design 3, dynamic
 * block-sparse causal attention): each head rates every (query tile, key
 * tile) pair by the dot product of the two tiles' mean-pooled q and k, and
 * keeps the best-rated key tiles beside a local window.
 *
 * top_k         key tiles kept by rating in every (head, query tile) row,
 *               chosen among the tiles the local window does not already
 *               keep; equal ratings go to the lower tile index; a row with
 *               fewer candidates keeps them all.  >= 0.
 * local_blocks  the local window: the key tiles overlapping the query tile's
 *               own key positions (the step's queries are the newest Nq of
 *               the n_keys keys, so query i sits at key n_keys - Nq + i),
 *               widened by local_blocks tiles on each side.  >= 0.
 */
typedef struct uf_topk_params {
  int32_t top_k;
  int32_t local_blocks;
} uf_topk_params;

/* Workspace bytes uf_block_mask_topk needs for Nq = n_q_tokens queries of
 * n_q_heads heads against any window of this cache description (fp32 tile
 * means of q and of the largest window's keys); 0 if the request is invalid. */
size_t uf_block_mask_workspace_bytes(const uf_kvcache_desc* desc, int32_t n_q_tokens, int32_t n_q_heads);

/*
 * Rate and select key tiles for a step's queries q ([Nq, Hq, head_dim] bf16,
 * Hq a multiple of n_kv_heads, Nq <= the window's n_keys) against the keys
 * the cache exposes now (call it after the step's append, before
 * uf_attn_step).  With an FP8 cache the keys are the stored codes times
 * k_scale; q is used as given (bf16, not quantized).
 * Tiles are 128 tokens in query order and in key order; the
 * last tile of each may be partial and is averaged over its own tokens.
 *
 * mask    device uint8 [Hq][ceil(Nq/128)][ceil(n_keys/128)], contiguous:
 *         1 = keep, 0 = skip.  It is a valid uf_block_mask with n_heads = Hq,
 *         stride_qblock = ceil(n_keys/128), stride_head = that times
 *         ceil(Nq/128).
 * scores  optional device float [same shape]: the ratings (plain dot
 *         products of the fp32 tile means, no 1/sqrt(d)); NULL = not written.
 * workspace  device memory of uf_block_mask_workspace_bytes bytes or more,
 *         256-byte aligned, used only during the call's kernels.
 * Means and ratings are fp32: each tile's rows summed in fp32, divided by
 * the row count; ratings are fma chains over head_dim in order.  At most
 * 3072 key tiles (UF_ERR_UNSUPPORTED beyond).  Nq == 0 is a no-op.  Two
 * kernel launches on `stream`; the cache state does not change.
 */
uf_status uf_block_mask_topk(const uf_tensor* q, const uf_kvcache* cache, const uf_topk_params* params,
                             uint8_t* mask, float* scores, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Static string naming a status code. */
const char* uf_status_string(uf_status status);

/* Detail of the calling thread's last failed call ("" if none). */
const char* uf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* UF_H */
