/* The C ABI of libuf driven from plain C, with no Python in the process: device memory from
 * the HIP runtime, a rolling cache with an anchor frame, appends that wrap the ring, attention
 * steps and one error path.  It checks what holds exactly, whatever the arithmetic:
 *   - a window of one key: every output row equals that key's value row, bit for bit;
 *   - an all-ones block mask gives the dense result bit for bit;
 *   - the allocation-free step equals the workspace step bit for bit (forced splits);
 *   - out overlapping q is refused with UF_ERR_INVALID_ARG, a message, no launch, and the
 *     window unchanged.
 * Exit status 0 and a last line "uf_c_check: ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "uf.h"

#define CHECK_HIP(x)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(2);                                                                         \
    }                                                                                  \
  } while (0)

#define CHECK_UF(x)                                                                         \
  do {                                                                                      \
    uf_status s_ = (x);                                                                     \
    if (s_ != UF_OK) {                                                                      \
      fprintf(stderr, "%s:%d: %s: %s (%s)\n", __FILE__, __LINE__, #x, uf_status_string(s_), \
              uf_last_error());                                                             \
      exit(3);                                                                              \
    }                                                                                       \
  } while (0)

static int failures = 0;

static void expect(int ok, const char* what) {
  printf("%s: %s\n", ok ? "pass" : "FAIL", what);
  if (!ok) ++failures;
}

/* seeded xorshift; bf16 bits of small values (sign, exponent 2^-3 .. 2^2, 7 random mantissa bits) */
static uint32_t rng = 12345u;
static uint16_t rand_bf16(void) {
  rng ^= rng << 13;
  rng ^= rng >> 17;
  rng ^= rng << 5;
  const uint32_t sign = (rng >> 31) & 1u, mant = rng & 0x7Fu, ex = 124u + (rng >> 8) % 6u;
  return (uint16_t)((sign << 15) | (ex << 7) | mant);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes));
  return p;
}

static void* dev_random(size_t n_elems) {
  uint16_t* h = (uint16_t*)malloc(n_elems * 2);
  for (size_t i = 0; i < n_elems; ++i) h[i] = rand_bf16();
  void* d = dev_alloc(n_elems * 2);
  CHECK_HIP(hipMemcpy(d, h, n_elems * 2, hipMemcpyHostToDevice));
  free(h);
  return d;
}

static uint16_t* to_host(const void* d, size_t n_elems) {
  uint16_t* h = (uint16_t*)malloc(n_elems * 2);
  CHECK_HIP(hipMemcpy(h, d, n_elems * 2, hipMemcpyDeviceToHost));
  return h;
}

static uf_tensor tensor(void* data, int n_tok, int heads, int d) {
  uf_tensor t;
  memset(&t, 0, sizeof t);
  t.data = data;
  t.dtype = UF_BF16;
  t.n_tokens = n_tok;
  t.n_heads = heads;
  t.head_dim = d;
  t.stride_token = (int64_t)heads * d;
  t.stride_head = d;
  return t;
}

/* A window of one key: softmax over one score is 1, so out = v exactly. */
static void single_key(void) {
  const int H = 2, HQ = 4, D = 128, NQ = 300;
  uf_kvcache_desc d;
  memset(&d, 0, sizeof d);
  d.n_kv_heads = H;
  d.head_dim = D;
  d.tokens_per_frame = 1;
  d.window_frames = 1;
  const size_t st = uf_kvcache_storage_bytes(&d);
  d.k_storage = dev_alloc(st);
  d.v_storage = dev_alloc(st);
  uf_kvcache* c = NULL;
  CHECK_UF(uf_kvcache_create(&d, &c));
  void* k = dev_random((size_t)H * D);
  void* v = dev_random((size_t)H * D);
  void* q = dev_random((size_t)NQ * HQ * D);
  void* o = dev_alloc((size_t)NQ * HQ * D * 2);
  uf_tensor tk = tensor(k, 1, H, D), tv = tensor(v, 1, H, D), tq = tensor(q, NQ, HQ, D), to = tensor(o, NQ, HQ, D);
  CHECK_UF(uf_kvcache_append(c, &tk, &tv, 1, 0, NULL));
  CHECK_UF(uf_attn_step(&tq, c, NULL, &to, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  uint16_t* hv = to_host(v, (size_t)H * D);
  uint16_t* ho = to_host(o, (size_t)NQ * HQ * D);
  int same = 1;
  for (int t = 0; t < NQ; ++t)
    for (int h = 0; h < HQ; ++h)
      for (int i = 0; i < D; ++i)
        same &= ho[((size_t)t * HQ + h) * D + i] == hv[(size_t)(h / (HQ / H)) * D + i];
  expect(same, "a single visible key returns its value row bit for bit (GQA 2)");
  free(hv);
  free(ho);
  CHECK_UF(uf_kvcache_destroy(c));
  hipFree(k); hipFree(v); hipFree(q); hipFree(o); hipFree(d.k_storage); hipFree(d.v_storage);
}

/* A stream over an anchor frame and a ring of 3 frames of 200 tokens: 6 appends of 2 frames
 * (the ring wraps), then dense vs all-ones mask, workspace vs static scratch, and an error. */
static void stream(void) {
  const int H = 2, HQ = 4, D = 128, L = 200, W = 4, A = 1, F = 2, NQ = F * L;
  uf_kvcache_desc d;
  memset(&d, 0, sizeof d);
  d.n_kv_heads = H;
  d.head_dim = D;
  d.tokens_per_frame = L;
  d.window_frames = W;
  d.anchor_frames = A;
  d.splits = 3;
  const size_t st = uf_kvcache_storage_bytes(&d);
  d.k_storage = dev_alloc(st);
  d.v_storage = dev_alloc(st);
  d.workspace_bytes = uf_attn_workspace_bytes(&d);
  d.workspace = dev_alloc(d.workspace_bytes);
  uf_kvcache* c = NULL;
  CHECK_UF(uf_kvcache_create(&d, &c));
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  void* q = dev_random((size_t)NQ * HQ * D);
  for (int step = 0; step < 6; ++step) {
    void* k = dev_random((size_t)NQ * H * D);
    void* v = dev_random((size_t)NQ * H * D);
    uf_tensor tk = tensor(k, NQ, H, D), tv = tensor(v, NQ, H, D);
    CHECK_UF(uf_kvcache_append(c, &tk, &tv, F, 0, s));
    CHECK_HIP(hipStreamSynchronize(s));
    hipFree(k);
    hipFree(v);
  }
  uf_window_info w;
  CHECK_UF(uf_kvcache_window(c, &w));
  expect(w.n_keys == (A + W) * L && w.anchor_keys == A * L, "window: anchor frame plus a full ring");

  const size_t n_out = (size_t)NQ * HQ * D;
  void* o_dense = dev_alloc(n_out * 2);
  void* o_mask = dev_alloc(n_out * 2);
  void* o_static = dev_alloc(n_out * 2);
  uf_tensor tq = tensor(q, NQ, HQ, D), t1 = tensor(o_dense, NQ, HQ, D), t2 = tensor(o_mask, NQ, HQ, D),
            t3 = tensor(o_static, NQ, HQ, D);
  const int nqb = (NQ + 127) / 128, nkb = (w.n_keys + 127) / 128;
  uint8_t* ones = (uint8_t*)malloc((size_t)nqb * nkb);
  memset(ones, 1, (size_t)nqb * nkb);
  uint8_t* dmask = (uint8_t*)dev_alloc((size_t)nqb * nkb);
  CHECK_HIP(hipMemcpy(dmask, ones, (size_t)nqb * nkb, hipMemcpyHostToDevice));
  uf_block_mask m;
  m.data = dmask;
  m.n_heads = 1;
  m.n_q_blocks = nqb;
  m.n_k_blocks = nkb;
  m.stride_head = (int64_t)nqb * nkb;
  m.stride_qblock = nkb;
  CHECK_UF(uf_attn_step(&tq, c, NULL, &t1, s));
  CHECK_UF(uf_attn_step(&tq, c, &m, &t2, s));
  CHECK_UF(uf_attn_step_static(&tq, c, NULL, &t3, s));
  CHECK_HIP(hipStreamSynchronize(s));
  uint16_t* h1 = to_host(o_dense, n_out);
  uint16_t* h2 = to_host(o_mask, n_out);
  uint16_t* h3 = to_host(o_static, n_out);
  expect(memcmp(h1, h2, n_out * 2) == 0, "an all-ones block mask gives the dense output bit for bit");
  expect(memcmp(h1, h3, n_out * 2) == 0, "the static-scratch step equals the workspace step (3 parts)");
  int finite = 1;
  for (size_t i = 0; i < n_out; ++i) finite &= ((h1[i] >> 7) & 0xFF) != 0xFF;
  expect(finite, "every output element is finite");

  /* out overlapping q: refused before any launch, message set, window unchanged */
  uf_window_info before, after;
  CHECK_UF(uf_kvcache_window(c, &before));
  const uf_status st_bad = uf_attn_step(&tq, c, NULL, &tq, s);
  CHECK_UF(uf_kvcache_window(c, &after));
  expect(st_bad == UF_ERR_INVALID_ARG && uf_last_error()[0] != '\0' &&
             memcmp(&before, &after, sizeof before) == 0,
         "out overlapping q is refused with UF_ERR_INVALID_ARG and a message");

  free(h1); free(h2); free(h3); free(ones);
  CHECK_HIP(hipStreamDestroy(s));
  CHECK_UF(uf_kvcache_destroy(c));
  hipFree(q); hipFree(o_dense); hipFree(o_mask); hipFree(o_static); hipFree(dmask);
  hipFree(d.k_storage); hipFree(d.v_storage); hipFree(d.workspace);
}

int main(void) {
  int n = 0;
  CHECK_HIP(hipGetDeviceCount(&n));
  if (n < 1) {
    fprintf(stderr, "uf_c_check: no GPU\n");
    return 4;
  }
  single_key();
  stream();
  if (failures) {
    printf("uf_c_check: %d check(s) failed\n", failures);
    return 1;
  }
  printf("uf_c_check: ok\n");
  return 0;
}
