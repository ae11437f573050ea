/* Every entry point's host path on the CPU, over the workload shapes and the
 * size limits, linked against host-only stand-ins of the kernel launchers
 * (tests/c/launch_stubs.cpp) and built with AddressSanitizer and
 * UndefinedBehaviorSanitizer: the validation, the split planning and the
 * assembly of launch arguments must neither touch memory out of bounds nor
 * hit undefined behaviour, and a refused call must launch nothing. */
#define _POSIX_C_SOURCE 200112L  /* setenv, unsetenv */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flashblock.h"

extern long long g_launches;

static int fails = 0;
#define CHECK(cond)                                                                \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "check failed: %s (line %d): %s\n", #cond, __LINE__, fb_last_error()); \
      ++fails;                                                                     \
    }                                                                              \
  } while (0)

#define FAKE ((void*)0x100000)
#define FF ((float*)0x100000)

/* head-major prefix [Hkv][T][D], contiguous block tensors */
static fb_desc make(int32_t dtype, int32_t b, int32_t hq, int32_t hkv, int32_t d, int32_t lb, const int64_t* off) {
  fb_desc x;
  memset(&x, 0, sizeof(x));
  x.abi_version = FB_ABI_VERSION;
  x.dtype = dtype;
  x.batch = b;
  x.hq = hq;
  x.hkv = hkv;
  x.head_dim = d;
  x.block_len = lb;
  x.prefix_offsets_host = off;
  x.prefix_offsets_dev = (const int64_t*)0x10000;
  x.q_stride_b = (int64_t)lb * hq * d;
  x.q_stride_t = (int64_t)hq * d;
  x.q_stride_h = d;
  x.kv_stride_b = (int64_t)lb * hkv * d;
  x.kv_stride_t = (int64_t)hkv * d;
  x.kv_stride_h = d;
  x.pre_stride_t = d;
  x.pre_stride_h = (off[b] > 0 ? off[b] : 1) * (int64_t)d;
  return x;
}

/* one shape through every entry point, fake device pointers; all must succeed */
static void every_call(const fb_desc* d, int with_sparse) {
  const size_t ws = fb_workspace_size(d, NULL);
  CHECK(ws >= 256);
  int32_t refreshed = -1;
  for (int32_t s = 0; s < 3; ++s) {
    CHECK(fb_step(d, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FF, FF, NULL, NULL, FAKE, FF, s, 2, FB_MODE_CACHED, 0,
                  &refreshed, FAKE, ws, NULL) == FB_OK);
    CHECK(refreshed == (s % 2 == 0));
    CHECK(fb_step_noalloc(d, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FF, FF, NULL, NULL, FAKE, FF, s, 2, FB_MODE_FULL, 0,
                          &refreshed, NULL) == FB_OK);
  }
  CHECK(fb_prefix_attn(d, FAKE, FAKE, FAKE, NULL, FF, FF, FAKE, ws, NULL) == FB_OK);
  CHECK(fb_prefix_partials(d, FAKE, FAKE, FAKE, NULL, FAKE, ws, NULL) == FB_OK);
  CHECK(fb_prefix_combine(d, NULL, FF, FF, FF, FF, FAKE, ws, NULL) == FB_OK);
  CHECK(fb_block_attn(d, FAKE, FAKE, FAKE, FF, FF, FAKE, FF, NULL) == FB_OK);
  CHECK(fb_refresh_mask_tau(d, FAKE, FAKE, FAKE, FAKE, 0.25f, 4, 1, (int32_t*)FAKE, (int32_t*)FAKE, FAKE, ws, NULL) == FB_OK);
  CHECK(fb_refresh_mask_gamma(d, FAKE, FAKE, 0.99f, 1, FF, (int32_t*)FAKE, NULL) == FB_OK);
  CHECK(fb_step_masked(d, FAKE, FAKE, FAKE, FAKE, FAKE, (int32_t*)FAKE, FF, FF, FAKE, FF, FAKE, ws, NULL) == FB_OK);
  CHECK(fb_append_block(d, FAKE, FAKE, FAKE, FAKE, (const int64_t*)FAKE, NULL) == FB_OK);
  if (with_sparse) {
    fb_sparse sp = {(const int32_t*)FAKE, 2, 64, FB_CHUNKS_SELECTED};
    const size_t wss = fb_workspace_size(d, &sp);
    CHECK(wss >= 256);
    for (int32_t s = 0; s < 2; ++s)
      CHECK(fb_step(d, FAKE, FAKE, FAKE, FAKE, FAKE, &sp, FF, FF, FF, FF, FAKE, FF, s, 2, FB_MODE_CACHED, 0, NULL,
                    FAKE, wss, NULL) == FB_OK);
    CHECK(fb_prefix_attn(d, FAKE, FAKE, FAKE, &sp, FF, FF, FAKE, wss, NULL) == FB_OK);
    const size_t sel_ws = fb_select_chunks_ws(d, 64);
    CHECK(sel_ws >= 256);
    CHECK(fb_select_chunks(d, FAKE, FAKE, 64, 2, (int32_t*)FAKE, FAKE, sel_ws, NULL) == FB_OK);
    CHECK(fb_pool_chunk_keys(d, FAKE, 64, 1 << 14, 0, FF, NULL) == FB_OK);
    CHECK(fb_select_chunks_pooled(d, FAKE, FF, 64, 1 << 14, 2, FF, (int32_t*)FAKE, NULL) == FB_OK);
  }
}

int main(void) {
  /* the workload shapes: tiny fp32, 32K MHA, 128K GQA, video, eight ragged ~64K streams */
  const int64_t off256[2] = {0, 256}, off32k[2] = {0, 32768}, off128k[2] = {0, 131072}, offv[2] = {0, 31200};
  int64_t off8[9] = {0};
  for (int b = 0; b < 8; ++b) off8[b + 1] = off8[b] + 65536 + (b % 3 - 1) * 9000 + b;
  fb_desc tiny = make(FB_F32, 1, 4, 4, 64, 16, off256);
  fb_desc mha = make(FB_BF16, 1, 32, 32, 128, 32, off32k);
  fb_desc gqa = make(FB_BF16, 1, 32, 8, 128, 64, off128k);
  fb_desc video = make(FB_BF16, 1, 12, 12, 128, 1560, offv);
  fb_desc batch8 = make(FB_BF16, 8, 32, 8, 128, 32, off8);
  every_call(&tiny, 0);
  every_call(&mha, 1);
  every_call(&gqa, 1);
  every_call(&video, 1);
  every_call(&batch8, 1);

  /* empty prefixes: all streams, and one of three */
  const int64_t off0[2] = {0, 0}, off3[4] = {0, 500, 500, 900};
  fb_desc empty = make(FB_BF16, 1, 8, 2, 64, 1, off0);
  every_call(&empty, 0);
  fb_desc holes = make(FB_BF16, 3, 8, 2, 64, 24, off3);
  every_call(&holes, 0);

  /* FB_DEBUG paths (the stand-in copy reports "no problem found") */
  setenv("FB_DEBUG", "1", 1);
  every_call(&gqa, 1);
  unsetenv("FB_DEBUG");

  /* limits: refused before anything is launched */
  long long before = g_launches;
  CHECK(fb_merge((int64_t)1 << 36, 128, FF, FF, FF, FF, FF, FF, NULL) == FB_OK);
  CHECK(g_launches == before + 1);
  before = g_launches;
  CHECK(fb_merge(((int64_t)1 << 36) + 1, 128, FF, FF, FF, FF, FF, FF, NULL) == FB_ERR_SHAPE);
  /* (stream, KV head) pairs beyond what one-workgroup-per-pair kernels launch */
  static int64_t offbig[(1 << 12) + 1];
  for (int b = 0; b <= (1 << 12); ++b) offbig[b] = (int64_t)b * 64;
  fb_desc many = make(FB_BF16, 1 << 12, 1024, 1024, 64, 1, offbig);
  CHECK(fb_workspace_size(&many, NULL) == 0);
  CHECK(fb_step(&many, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FF, FF, NULL, NULL, FAKE, NULL, 0, 1, FB_MODE_CACHED, 0,
                NULL, FAKE, (size_t)1 << 40, NULL) == FB_ERR_SHAPE);
  /* passes past the attention grid limit: 2^21 (stream, KV head) pairs with 512 query rows each
     (four prefix row tiles, sixteen block row tiles) */
  fb_desc wide = make(FB_BF16, 1 << 12, 2048, 512, 64, 128, offbig);
  CHECK(fb_step(&wide, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FF, FF, NULL, NULL, FAKE, NULL, 0, 1, FB_MODE_CACHED, 0,
                NULL, FAKE, (size_t)1 << 40, NULL) == FB_ERR_SHAPE);
  CHECK(fb_block_attn(&wide, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL) == FB_ERR_SHAPE);
  /* the no-allocation step beyond its scratch */
  const int64_t off8k[9] = {0, 4096, 8192, 12288, 16384, 20480, 24576, 28672, 32768};
  fb_desc big = make(FB_BF16, 8, 64, 1, 128, 1024, off8k);
  CHECK(fb_workspace_size(&big, NULL) > FB_NOALLOC_SCRATCH_BYTES);
  CHECK(fb_step_noalloc(&big, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FF, FF, NULL, NULL, FAKE, NULL, 0, 1,
                        FB_MODE_CACHED, 0, NULL, NULL) == FB_ERR_WORKSPACE);
  CHECK(g_launches == before);

  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("host_paths ok (%lld launches checked)\n", g_launches);
  return 0;
}
