/* Plain C99 client of libflashblock.so: the header compiles as C, the
 * library links and answers its validation paths without a GPU. */
#include <stdio.h>
#include <string.h>

#include "flashblock.h"

static int fails = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

int main(void) {
  CHECK(fb_abi_version() == FB_ABI_VERSION);
  CHECK(strcmp(fb_status_string(FB_ERR_WORKSPACE), "workspace too small") == 0);

  /* 128K-token GQA layer: 32 query heads over 8 KV heads, D 128, block 64, head-major prefix */
  const int64_t off[2] = {0, 131072};
  fb_desc d;
  memset(&d, 0, sizeof(d));
  d.abi_version = FB_ABI_VERSION;
  d.dtype = FB_BF16;
  d.batch = 1;
  d.hq = 32;
  d.hkv = 8;
  d.head_dim = 128;
  d.block_len = 64;
  d.prefix_offsets_host = off;
  d.prefix_offsets_dev = (const int64_t*)0x10000; /* never dereferenced by validation */
  d.q_stride_b = 64 * 32 * 128;
  d.q_stride_t = 32 * 128;
  d.q_stride_h = 128;
  d.kv_stride_b = 64 * 8 * 128;
  d.kv_stride_t = 8 * 128;
  d.kv_stride_h = 128;
  d.pre_stride_t = 128;
  d.pre_stride_h = 131072 * 128;
  const size_t ws = fb_workspace_size(&d, NULL);
  /* 32 splits of 64 tiles, then 256 bytes for a masked step's unit plan */
  CHECK(ws == (size_t)32 * 32 * 64 * 128 * 4 + (size_t)32 * 32 * 64 * 4 + 256);

  void* fake = (void*)0x100000;
  float* ff = (float*)fake;
  int32_t refreshed = -1;
  /* r = 0 is rejected before anything is launched, and nothing is written */
  CHECK(fb_step(&d, fake, fake, fake, fake, fake, NULL, ff, ff, NULL, NULL, fake, NULL, 0, 0, FB_MODE_CACHED, 0,
                &refreshed, fake, ws, NULL) == FB_ERR_ARG);
  CHECK(refreshed == -1);
  CHECK(strlen(fb_last_error()) > 0);
  /* a workspace one byte short */
  CHECK(fb_step(&d, fake, fake, fake, fake, fake, NULL, ff, ff, NULL, NULL, fake, NULL, 0, 8, FB_MODE_CACHED, 0,
                NULL, fake, ws - 1, NULL) == FB_ERR_WORKSPACE);
  /* hq not a multiple of hkv */
  d.hq = 30;
  CHECK(fb_workspace_size(&d, NULL) == 0);
  CHECK(fb_prefix_attn(&d, fake, fake, fake, NULL, ff, ff, fake, ws, NULL) == FB_ERR_SHAPE);
  d.hq = 32;
  /* chunk selection: more chunks asked for than the stream has */
  int32_t* idx = (int32_t*)fake;
  CHECK(fb_select_chunks(&d, fake, fake, 64, 4096, idx, fake, fb_select_chunks_ws(&d, 64), NULL) == FB_ERR_ARG);
  /* the merge with zero rows is a no-op */
  CHECK(fb_merge(0, 128, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == FB_OK);

  if (fails) return 1;
  printf("abi_smoke ok\n");
  return 0;
}
