// Host side of libflashblock.so: argument validation, split planning and the
// C ABI declared in include/flashblock.h.  Every check runs before anything is
// enqueued; the library allocates nothing and keeps no state between calls.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "fb_internal.h"
#include "flashblock.h"

static_assert(fb::kDtypeBf16 == FB_BF16, "dtype tag of the kernels");
static_assert(fb::kNoAllocScratchBytes == FB_NOALLOC_SCRATCH_BYTES, "no-allocation scratch size");

namespace {

thread_local char g_err[512] = "";

fb_status fail(fb_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

// MI355X: 256 compute units.  Split planning targets whole waves of
// workgroups over them; the constant keeps plans (and workspace sizes)
// independent of the calling thread's device state.
constexpr int kCUs = 256;
constexpr int kMinSplitTiles = 4;  // >= 256 keys per split
constexpr size_t kAlign = 256;
// Launch limits: an attention grid of at most kMaxAttnWorkgroups workgroups of
// up to 512 threads, and at most kMaxStreamHeads (stream, KV head) pairs, keep
// every dispatch's work-item count inside its 32-bit limit.
constexpr int64_t kMaxAttnWorkgroups = 1LL << 22;
constexpr int64_t kMaxStreamHeads = 1LL << 21;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize(const fb_desc* d) { return d->dtype == FB_BF16 ? 2 : 4; }

// Kernel configuration of each pass, by query rows per KV head (G * Lb).
int prefix_cfg(const fb_desc* d) {
  const int rows = (d->hq / d->hkv) * d->block_len;
#if defined(FB_PREFIX_CFG_32) && defined(FB_PREFIX_CFG_64) && defined(FB_PREFIX_CFG_128) && defined(FB_PREFIX_CFG_256)
  // build-time override of the per-size choice (used to sweep configurations)
  return rows <= 32 ? FB_PREFIX_CFG_32 : rows <= 64 ? FB_PREFIX_CFG_64 : rows <= 128 ? FB_PREFIX_CFG_128
                                                                                     : FB_PREFIX_CFG_256;
#else
  // measured on MI355X: two independent workgroups per CU, each 2-stage
  // (their waves drift apart, so one's softmax overlaps the other's MFMAs);
  // up to 64 rows four 16-row waves, also for 32 rows, where the upper two
  // only issue tile loads: every wave then issues half the loads, and the
  // pass runs 5-8% faster than with two waves.  Above 128 rows, 256-row
  // tiles of one 8-wave workgroup each fetch every KV tile once per 256 rows:
  // 5% faster at 256 rows (128K GQA, where the board's power cap sets the
  // clock and the halved HBM and DMA traffic buys clock), 6% on the
  // 1560-row video prefix (MFMA-bound) despite its longer padded last tile.
  // They are taken unless they pad more than an eighth beyond 128-row tiles.
  if (rows <= 64) return fb::CFG_P64_X2;
  if (rows <= 128) return fb::CFG_P128_X2;
  const int64_t pad256 = ceil_div(rows, 256) * 256, pad128 = ceil_div(rows, 128) * 128;
  return pad256 * 8 <= pad128 * 9 ? fb::CFG_P256 : fb::CFG_P128_X2;
#endif
}
int block_cfg(const fb_desc* d) {
  const int rows = (d->hq / d->hkv) * d->block_len;
  const bool key_groups = rows >= 1024 || d->block_len >= 512;
#if defined(FB_BLOCK_CFG_BIG) && defined(FB_BLOCK_CFG_SMALL)
  // build-time override (used to sweep configurations)
  return key_groups ? FB_BLOCK_CFG_BIG : FB_BLOCK_CFG_SMALL;
#else
  // measured on MI355X: blocks of 1024 rows and more per KV head, and
  // blocks of 512 keys and more, take workgroups in two key groups: 64 rows
  // (four 32-row waves, two workgroups per CU) or 80 rows (ten 16-row waves,
  // one per CU).  80 rows wherever they need fewer workgroups per CU than 64
  // rows: the 1560-row video frame, 240 workgroups against 300, 25.3 against
  // 29.8 us; two frames, 480 against 600, 49.3 against 53.6.  With as many
  // per CU, the two concurrent 64-row workgroups win (32 heads x 768
  // tokens, 384 against 320: 19.1 against 28.5 us; 8 heads x 1560, 200
  // against 160: 24.1 against 24.5).  Against the 32-row text workgroups,
  // key groups gain 9-33% from 512 keys up (32 x 768 tokens: 28.3 -> 19.1
  // us) and lose below 200 (GQA 32/8 x 160 tokens: 6.9 -> 8.0).
  // Text blocks are latency-bound and run fastest on
  // 4-wave workgroups whose extra waves only issue tile loads: 16 rows (one
  // row wave) while that gives at most one workgroup per CU, else 32 rows
  // (two row waves), which beat 16-row ones once those fill the CUs twice.
  if (key_groups) {
    const int64_t wgs64 = (int64_t)d->batch * d->hkv * ceil_div(rows, 64);
    const int64_t wgs80 = (int64_t)d->batch * d->hkv * ceil_div(rows, 80);
    return ceil_div(wgs80, kCUs) < ceil_div(wgs64, kCUs) ? fb::CFG_B80_K2 : fb::CFG_B64_K2;
  }
  const int64_t wgs16 = (int64_t)d->batch * d->hkv * ceil_div(rows, 16);
  return wgs16 <= kCUs ? fb::CFG_B16_LD : fb::CFG_B32_LD;
#endif
}
// fp32 inputs run the fp32 MFMA kernel: 64 rows per workgroup (4 waves x 16), 2 per CU.
fb::CfgInfo pass_info(const fb_desc* d, int cfg) {
  if (d->dtype == FB_F32) return {64, 2};
  return fb::cfg_info(cfg);
}

fb_status check_desc(const fb_desc* d) {
  if (!d) return fail(FB_ERR_NULL, "fb_desc is NULL");
  if (d->abi_version != FB_ABI_VERSION)
    return fail(FB_ERR_ARG, "abi_version %d != %d", d->abi_version, FB_ABI_VERSION);
  if (d->dtype != FB_F32 && d->dtype != FB_BF16)
    return fail(FB_ERR_UNSUPPORTED, "dtype %d not supported (FB_F32, FB_BF16)", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(FB_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", d->head_dim);
  if (d->batch < 1 || d->hq < 1 || d->hkv < 1 || d->block_len < 1)
    return fail(FB_ERR_SHAPE, "batch, hq, hkv and block_len must be >= 1 (got %d, %d, %d, %d)", d->batch,
                d->hq, d->hkv, d->block_len);
  if (d->hq % d->hkv != 0) return fail(FB_ERR_SHAPE, "hq %d is not a multiple of hkv %d", d->hq, d->hkv);
  // kernels with one workgroup per (stream, KV head) launch up to 1024 threads
  // each: the grid's work-item count stays inside 32 bits
  if ((int64_t)d->batch * d->hkv > kMaxStreamHeads)
    return fail(FB_ERR_SHAPE, "batch * hkv = %lld > %lld", (long long)d->batch * d->hkv, (long long)kMaxStreamHeads);
  const int64_t rows = (int64_t)d->batch * d->hq * d->block_len;
  if (rows > (1LL << 30) || (int64_t)(d->hq / d->hkv) * d->block_len > (1 << 24))
    return fail(FB_ERR_SHAPE, "batch * hq * block_len too large");
  if (!isfinite(d->softmax_scale)) return fail(FB_ERR_ARG, "softmax_scale is not finite");
  const int64_t e = esize(d);
  const int64_t strides[] = {d->q_stride_b, d->q_stride_t, d->q_stride_h, d->kv_stride_b, d->kv_stride_t,
                             d->kv_stride_h, d->pre_stride_t, d->pre_stride_h};
  for (int64_t s : strides) {
    if (s < 0) return fail(FB_ERR_SHAPE, "negative stride %lld", (long long)s);
    if ((s * e) % 16 != 0)
      return fail(FB_ERR_ALIGN, "stride %lld elements is not a multiple of 16 bytes", (long long)s);
  }
  // a 64-key tile's row offsets are kept in 31 bits by the kernels
  if (d->kv_stride_t * e * 64 >= (1LL << 31) || d->pre_stride_t * e * 64 >= (1LL << 31))
    return fail(FB_ERR_SHAPE, "token stride too large");
  return FB_OK;
}

int64_t total_prefix(const fb_desc* d) { return d->prefix_offsets_host[d->batch] - d->prefix_offsets_host[0]; }

fb_status check_offsets(const fb_desc* d) {
  if (!d->prefix_offsets_host || !d->prefix_offsets_dev)
    return fail(FB_ERR_NULL, "prefix_offsets_host and prefix_offsets_dev are required");
  const int64_t* o = d->prefix_offsets_host;
  if (o[0] < 0) return fail(FB_ERR_SHAPE, "prefix offset[0] = %lld < 0", (long long)o[0]);
  for (int b = 0; b < d->batch; ++b) {
    if (o[b + 1] < o[b])
      return fail(FB_ERR_SHAPE, "prefix offsets decrease at stream %d (%lld -> %lld)", b, (long long)o[b],
                  (long long)o[b + 1]);
    if (o[b + 1] - o[b] > (1LL << 30)) return fail(FB_ERR_SHAPE, "prefix of stream %d too long", b);
  }
  return FB_OK;
}

fb_status check_sparse(const fb_sparse* sp, bool need_mode) {
  if (!sp) return FB_OK;
  if (!sp->chunk_idx_dev) return fail(FB_ERR_NULL, "fb_sparse.chunk_idx_dev is NULL");
  if (sp->k < 1) return fail(FB_ERR_ARG, "fb_sparse.k = %d < 1", sp->k);
  if (sp->chunk_len < 64 || sp->chunk_len % 64 != 0)
    return fail(FB_ERR_ARG, "fb_sparse.chunk_len = %d is not a positive multiple of 64", sp->chunk_len);
  if (need_mode && sp->mode != FB_CHUNKS_SELECTED && sp->mode != FB_CHUNKS_COMPLEMENT)
    return fail(FB_ERR_ARG, "fb_sparse.mode = %d (FB_CHUNKS_SELECTED or FB_CHUNKS_COMPLEMENT)", sp->mode);
  if ((int64_t)sp->k * (sp->chunk_len / 64) > (1 << 28)) return fail(FB_ERR_ARG, "fb_sparse.k too large");
  return FB_OK;
}

// ---------------------------------------------------------------------------
// split plan of the prefix pass
// ---------------------------------------------------------------------------

struct PrefixPlan {
  int cfg, row_tiles, split_tiles, total_splits, n_work, grid;
  int chunk_mode, n_sel, chunk_tiles;
  size_t part_o_bytes, part_lse_bytes;
};

int64_t logical_tiles_host(const fb_desc* d, int b, int chunk_mode, int n_sel, int chunk_tiles) {
  if (chunk_mode == fb::CHUNKS_SELECTED) return (int64_t)n_sel * chunk_tiles;
  const int64_t lp = d->prefix_offsets_host[b + 1] - d->prefix_offsets_host[b];
  return ceil_div(lp, fb::kTile);
}

fb_status plan_prefix(const fb_desc* d, int chunk_mode, int n_sel, int chunk_len, PrefixPlan* p) {
  const int rows = (d->hq / d->hkv) * d->block_len;
  p->cfg = prefix_cfg(d);
  const fb::CfgInfo ci = pass_info(d, p->cfg);
  p->row_tiles = (int)ceil_div(rows, ci.rows);
  p->chunk_mode = chunk_mode;
  p->n_sel = n_sel;
  p->chunk_tiles = chunk_mode == fb::CHUNKS_ALL ? 1 : chunk_len / fb::kTile;
  const int64_t units = (int64_t)d->hkv * p->row_tiles;
  int64_t total_tiles = 0;
  for (int b = 0; b < d->batch; ++b) total_tiles += logical_tiles_host(d, b, chunk_mode, n_sel, p->chunk_tiles);
  // Smallest split length whose workgroups all fit in one resident round
  // (capacity = CUs x workgroups per CU): a second, partly filled round would
  // double the pass time.  Splits of at least kMinSplitTiles tiles (bf16).
  const int64_t capacity = (int64_t)kCUs * ci.wgs_per_cu;
  int64_t max_tiles = 0;
  for (int b = 0; b < d->batch; ++b)
    max_tiles = std::max(max_tiles, logical_tiles_host(d, b, chunk_mode, n_sel, p->chunk_tiles));
  auto wgs_for = [&](int64_t st_) {
    int64_t n = 0;
    for (int b = 0; b < d->batch; ++b) n += ceil_div(logical_tiles_host(d, b, chunk_mode, n_sel, p->chunk_tiles), st_);
    return n * units;
  };
  // (fp32 keeps splits of one tile: more workgroups for its small shapes)
  const int64_t min_split = d->dtype == FB_F32 ? 1 : kMinSplitTiles;
  int64_t st = std::max<int64_t>(min_split, ceil_div(total_tiles * units, capacity));
  while (st < max_tiles && wgs_for(st) > capacity) ++st;
  st = std::max<int64_t>(st, min_split);
  if (st > (1 << 28)) st = 1 << 28;
  p->split_tiles = (int)st;
  int64_t splits = 0;
  for (int b = 0; b < d->batch; ++b)
    splits += ceil_div(logical_tiles_host(d, b, chunk_mode, n_sel, p->chunk_tiles), st);
  const int64_t work = splits * units;
  if (work > kMaxAttnWorkgroups)
    return fail(FB_ERR_SHAPE, "prefix pass needs %lld workgroups > %lld", (long long)work,
                (long long)kMaxAttnWorkgroups);
  p->total_splits = (int)splits;
  p->n_work = (int)work;
  p->grid = (int)ceil_div(work, 8) * 8;
  const size_t prow = (size_t)splits * d->hq * d->block_len;
  p->part_o_bytes = align_up(prow * d->head_dim * sizeof(float));
  p->part_lse_bytes = align_up(prow * sizeof(float));
  return FB_OK;
}

float c_log2(const fb_desc* d) {
  const float scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  return scale * 1.4426950408889634f;
}

void fill_common(const fb_desc* d, const void* q, fb::AttnArgs* a) {
  memset(a, 0, sizeof(*a));
  a->q = q;
  a->q_sb = d->q_stride_b;
  a->q_st = d->q_stride_t;
  a->q_sh = d->q_stride_h;
  a->B = d->batch;
  a->Hq = d->hq;
  a->Hkv = d->hkv;
  a->G = d->hq / d->hkv;
  a->Lb = d->block_len;
  a->rows = a->G * d->block_len;
  a->c_log2 = c_log2(d);
}

fb_status hip_status(int err, const char* what) {
  if (err != 0) return fail(FB_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
  return FB_OK;
}

// The two halves of the prefix pass for a chosen chunk mode.  Both derive the
// same plan (and so the same workspace layout) from (d, chunk mode, sp).
fb_status run_partials(const fb_desc* d, const void* q, const void* k_pre, const void* v_pre, int chunk_mode,
                       const fb_sparse* sp, void* ws, size_t ws_bytes, void* stream,
                       const int32_t* unit_plan = nullptr) {
  PrefixPlan p;
  const int n_sel = sp ? sp->k : 0;
  fb_status st = plan_prefix(d, chunk_mode, n_sel, sp ? sp->chunk_len : 64, &p);
  if (st != FB_OK) return st;
  if (p.part_o_bytes + p.part_lse_bytes > ws_bytes)
    return fail(FB_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.part_o_bytes + p.part_lse_bytes);
  fb::AttnArgs a;
  fill_common(d, q, &a);
  a.k = k_pre;
  a.v = v_pre;
  a.kv_st = d->pre_stride_t;
  a.kv_sh = d->pre_stride_h;
  a.offsets = d->prefix_offsets_dev;
  a.split_tiles = p.split_tiles;
  a.row_tiles = p.row_tiles;
  a.n_work = p.n_work;
  a.grid = p.grid;
  a.chunks = sp ? sp->chunk_idx_dev : nullptr;
  a.n_sel = n_sel;
  a.chunk_tiles = p.chunk_tiles;
  a.chunk_mode = chunk_mode;
  a.part_o = (float*)ws;
  a.part_lse = (float*)((char*)ws + p.part_o_bytes);
  a.plan = unit_plan;
  return hip_status(fb::launch_attn(a, d->dtype, d->head_dim, p.cfg, true, stream), "prefix attention launch");
}

fb_status run_combine(const fb_desc* d, int chunk_mode, const fb_sparse* sp, const float* extra_o,
                      const float* extra_lse, float* o_ext, float* lse_ext, const void* ws, size_t ws_bytes,
                      void* stream, const int32_t* unit_plan = nullptr) {
  PrefixPlan p;
  const int n_sel = sp ? sp->k : 0;
  fb_status st = plan_prefix(d, chunk_mode, n_sel, sp ? sp->chunk_len : 64, &p);
  if (st != FB_OK) return st;
  if (p.part_o_bytes + p.part_lse_bytes > ws_bytes)
    return fail(FB_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.part_o_bytes + p.part_lse_bytes);
  fb::CombineArgs c;
  memset(&c, 0, sizeof(c));
  c.part_o = (const float*)ws;
  c.part_lse = (const float*)((const char*)ws + p.part_o_bytes);
  c.offsets = d->prefix_offsets_dev;
  c.B = d->batch;
  c.Hq = d->hq;
  c.Lb = d->block_len;
  c.D = d->head_dim;
  c.split_tiles = p.split_tiles;
  c.n_sel = n_sel;
  c.chunk_tiles = p.chunk_tiles;
  c.chunk_mode = chunk_mode;
  c.total_splits = p.total_splits;
  c.extra_o = extra_o;
  c.extra_lse = extra_lse;
  c.o = o_ext;
  c.lse = lse_ext;
  c.plan = unit_plan;
  // a unit plan packs G * Lb rows per unit: the workspace holds Hkv units per split of the all-heads plan
  if (unit_plan) c.total_splits = p.total_splits * d->hkv;
  c.Hkv = d->hkv;
  c.G = d->hq / d->hkv;
  c.max_splits = 0;
  for (int b = 0; b < d->batch; ++b)
    c.max_splits = (int32_t)std::max<int64_t>(c.max_splits, ceil_div(logical_tiles_host(d, b, chunk_mode, n_sel,
                                                                                        p.chunk_tiles), p.split_tiles));
  if (unit_plan) c.max_splits = p.total_splits * d->hkv;   // the plan's split lengths are decided on the device
  const int64_t rows = (int64_t)d->batch * d->hq * d->block_len;
  return hip_status(fb::launch_combine(c, rows, stream), "split combine launch");
}

fb_status run_prefix(const fb_desc* d, const void* q, const void* k_pre, const void* v_pre, int chunk_mode,
                     const fb_sparse* sp, const float* extra_o, const float* extra_lse, float* o_ext,
                     float* lse_ext, void* ws, size_t ws_bytes, void* stream, const int32_t* unit_plan = nullptr) {
  fb_status st = run_partials(d, q, k_pre, v_pre, chunk_mode, sp, ws, ws_bytes, stream, unit_plan);
  if (st != FB_OK) return st;
  return run_combine(d, chunk_mode, sp, extra_o, extra_lse, o_ext, lse_ext, ws, ws_bytes, stream, unit_plan);
}

// Workgroups of the block pass: (stream, KV head, row tile).
int64_t block_work(const fb_desc* d, int cfg) {
  const int64_t rows = (int64_t)(d->hq / d->hkv) * d->block_len;
  return (int64_t)d->batch * d->hkv * ceil_div(rows, pass_info(d, cfg).rows);
}

// Every plan a call will launch, checked before anything is launched: the
// prefix pass in the chunk modes it runs (dense, or both sparse modes), and
// the block pass.
fb_status check_plans(const fb_desc* d, const fb_sparse* sp, bool prefix, bool block) {
  PrefixPlan p;
  if (prefix) {
    if (!sp) {
      fb_status st = plan_prefix(d, fb::CHUNKS_ALL, 0, 64, &p);
      if (st != FB_OK) return st;
    } else {
      for (int mode : {fb::CHUNKS_SELECTED, fb::CHUNKS_COMPLEMENT}) {
        fb_status st = plan_prefix(d, mode, sp->k, sp->chunk_len, &p);
        if (st != FB_OK) return st;
      }
    }
  }
  if (block) {
    const int64_t work = block_work(d, block_cfg(d));
    if (work > kMaxAttnWorkgroups)
      return fail(FB_ERR_SHAPE, "block pass needs %lld workgroups > %lld", (long long)work,
                  (long long)kMaxAttnWorkgroups);
  }
  return FB_OK;
}

fb_status run_block(const fb_desc* d, const void* q, const void* k_blk, const void* v_blk, const float* o_ext,
                    const float* lse_ext, void* o, float* lse_out, void* stream) {
  fb::AttnArgs a;
  fill_common(d, q, &a);
  a.k = k_blk;
  a.v = v_blk;
  a.kv_sb = d->kv_stride_b;
  a.kv_st = d->kv_stride_t;
  a.kv_sh = d->kv_stride_h;
  a.offsets = nullptr;
  const int cfg = block_cfg(d);
  a.row_tiles = (int)ceil_div(a.rows, pass_info(d, cfg).rows);
  a.split_tiles = (int)ceil_div(d->block_len, fb::kTile);
  const int64_t work = block_work(d, cfg);   // within kMaxAttnWorkgroups: check_plans ran first
  a.n_work = (int)work;
  a.grid = (int)ceil_div(work, 8) * 8;
  a.ext_o = o_ext;
  a.ext_lse = lse_ext;
  a.o = o;
  a.lse_out = lse_out;
  return hip_status(fb::launch_attn(a, d->dtype, d->head_dim, cfg, false, stream), "block attention launch");
}

// Bytes of a masked step's unit plan, kept after the all-heads plan's partials.
size_t unit_plan_bytes(const fb_desc* d) { return align_up((size_t)fb::plan_ints((int64_t)d->batch * d->hkv) * 4); }

size_t workspace_for(const fb_desc* d, const fb_sparse* sp) {
  PrefixPlan p;
  size_t need = 0;
  if (!sp) {
    if (plan_prefix(d, fb::CHUNKS_ALL, 0, 64, &p) != FB_OK) return 0;
    need = p.part_o_bytes + p.part_lse_bytes + unit_plan_bytes(d);   // fb_step_masked: partials + plan
  } else {
    for (int mode : {fb::CHUNKS_SELECTED, fb::CHUNKS_COMPLEMENT}) {
      if (plan_prefix(d, mode, sp->k, sp->chunk_len, &p) != FB_OK) return 0;
      need = std::max(need, p.part_o_bytes + p.part_lse_bytes);
    }
  }
  need = std::max(need, (size_t)d->batch * d->block_len * sizeof(int32_t));   // fb_refresh_mask_tau flags
  return std::max<size_t>(need, kAlign);
}

fb_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return fail(FB_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!ws) return fail(FB_ERR_NULL, "workspace is NULL");
  if (((uintptr_t)ws % kAlign) != 0) return fail(FB_ERR_ALIGN, "workspace is not 256-byte aligned");
  return FB_OK;
}

}  // namespace

// FB_DEBUG=1 in the environment turns on the checks below: a reuse step's cache
// is scanned for NaN, and sparse chunk lists are checked against their contract.
static bool debug_checks() {
  const char* e = getenv("FB_DEBUG");
  return e && e[0] == '1' && e[1] == '\0';
}

// The debug check waits on the stream, which a stream under graph capture
// cannot do: it is skipped there.
static bool capturing(void* stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing((hipStream_t)stream, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

// Debug check before a reuse step: scans the cached partial (O, then LSE)
// for NaN, with the flag in the first word of the workspace, and waits for
// the answer on the stream.
static fb_status cache_has_nan(const fb_desc* d, const float* oc, const float* lc, void* ws, int32_t step,
                               void* stream) {
  const int64_t rows = (int64_t)d->batch * d->hq * d->block_len;
  int32_t* flag = (int32_t*)ws;
  int rc = fb::launch_nan_scan(oc, rows * d->head_dim, flag, true, stream);
  if (rc == 0) rc = fb::launch_nan_scan(lc, rows, flag, false, stream);
  int32_t host = 0;
  if (rc == 0) rc = (int)hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (rc == 0) rc = (int)hipStreamSynchronize((hipStream_t)stream);
  fb_status st = hip_status(rc, "FB_DEBUG cache check");
  if (st != FB_OK) return st;
  if (host) return fail(FB_ERR_ARG, "reuse step %d: the cached partial holds NaN (was it written by a refresh step of this block?)", step);
  return FB_OK;
}

// Debug check of a sparse chunk list (ascending, unique, in range for its
// stream), with the flag in the first word of the workspace; waits for the
// answer on the stream.
static fb_status chunk_list_bad(const fb_desc* d, const fb_sparse* sp, void* ws, void* stream) {
  int32_t* flag = (int32_t*)ws;
  int rc = fb::launch_chunk_check(sp->chunk_idx_dev, d->prefix_offsets_dev, d->batch, d->hkv, sp->k, sp->chunk_len,
                                  flag, stream);
  int32_t host = 0;
  if (rc == 0) rc = (int)hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (rc == 0) rc = (int)hipStreamSynchronize((hipStream_t)stream);
  fb_status st = hip_status(rc, "FB_DEBUG chunk list check");
  if (st != FB_OK) return st;
  if (host)
    return fail(FB_ERR_ARG, "fb_sparse.chunk_idx_dev: a (stream, KV head) list is not ascending and unique, or "
                "names a chunk outside its stream's prefix");
  return FB_OK;
}

static fb_status debug_chunk_check(const fb_desc* d, const fb_sparse* sp, void* ws, void* stream) {
  if (!sp || !debug_checks() || capturing(stream)) return FB_OK;
  return chunk_list_bad(d, sp, ws, stream);
}

extern "C" {

int32_t fb_abi_version(void) { return FB_ABI_VERSION; }

const char* fb_last_error(void) { return g_err; }

const char* fb_status_string(fb_status s) {
  switch (s) {
    case FB_OK: return "ok";
    case FB_ERR_NULL: return "null pointer";
    case FB_ERR_SHAPE: return "bad shape";
    case FB_ERR_ALIGN: return "misaligned pointer or stride";
    case FB_ERR_WORKSPACE: return "workspace too small";
    case FB_ERR_UNSUPPORTED: return "unsupported dtype or head_dim";
    case FB_ERR_ARG: return "bad argument";
    case FB_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t fb_workspace_size(const fb_desc* d, const fb_sparse* sp) {
  clear_error();
  if (check_desc(d) != FB_OK || check_offsets(d) != FB_OK || check_sparse(sp, false) != FB_OK ||
      check_plans(d, sp, true, false) != FB_OK)
    return 0;
  return workspace_for(d, sp);
}

fb_status fb_prefix_attn(const fb_desc* d, const void* q_blk, const void* k_pre, const void* v_pre,
                         const fb_sparse* sp, float* o_ext, float* lse_ext, void* ws, size_t ws_bytes,
                         void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st == FB_OK) st = check_offsets(d);
  if (st == FB_OK) st = check_sparse(sp, true);
  if (st == FB_OK) st = check_plans(d, sp, true, false);
  if (st != FB_OK) return st;
  if (!q_blk || !o_ext || !lse_ext) return fail(FB_ERR_NULL, "q_blk, o_ext and lse_ext are required");
  if (total_prefix(d) > 0 && (!k_pre || !v_pre))
    return fail(FB_ERR_NULL, "k_pre and v_pre are required for a non-empty prefix");
  if (!aligned16(q_blk) || !aligned16(k_pre) || !aligned16(v_pre) || !aligned16(o_ext))
    return fail(FB_ERR_ALIGN, "q_blk, k_pre, v_pre and o_ext must be 16-byte aligned");
  const size_t need = workspace_for(d, sp);
  st = check_ws(ws, ws_bytes, need);
  if (st != FB_OK) return st;
  st = debug_chunk_check(d, sp, ws, stream);
  if (st != FB_OK) return st;
  const int mode = sp ? sp->mode : fb::CHUNKS_ALL;
  return run_prefix(d, q_blk, k_pre, v_pre, mode, sp, nullptr, nullptr, o_ext, lse_ext, ws, ws_bytes, stream);
}

fb_status fb_prefix_partials(const fb_desc* d, const void* q_blk, const void* k_pre, const void* v_pre,
                             const fb_sparse* sp, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st == FB_OK) st = check_offsets(d);
  if (st == FB_OK) st = check_sparse(sp, true);
  if (st == FB_OK) st = check_plans(d, sp, true, false);
  if (st != FB_OK) return st;
  if (!q_blk) return fail(FB_ERR_NULL, "q_blk is required");
  if (total_prefix(d) > 0 && (!k_pre || !v_pre))
    return fail(FB_ERR_NULL, "k_pre and v_pre are required for a non-empty prefix");
  if (!aligned16(q_blk) || !aligned16(k_pre) || !aligned16(v_pre))
    return fail(FB_ERR_ALIGN, "q_blk, k_pre and v_pre must be 16-byte aligned");
  st = check_ws(ws, ws_bytes, workspace_for(d, sp));
  if (st == FB_OK) st = debug_chunk_check(d, sp, ws, stream);
  if (st != FB_OK) return st;
  return run_partials(d, q_blk, k_pre, v_pre, sp ? sp->mode : fb::CHUNKS_ALL, sp, ws, ws_bytes, stream);
}

fb_status fb_prefix_combine(const fb_desc* d, const fb_sparse* sp, const float* extra_o, const float* extra_lse,
                            float* o_ext, float* lse_ext, const void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st == FB_OK) st = check_offsets(d);
  if (st == FB_OK) st = check_sparse(sp, true);
  if (st == FB_OK) st = check_plans(d, sp, true, false);
  if (st != FB_OK) return st;
  if (!o_ext || !lse_ext) return fail(FB_ERR_NULL, "o_ext and lse_ext are required");
  if ((extra_o == nullptr) != (extra_lse == nullptr))
    return fail(FB_ERR_NULL, "extra_o and extra_lse must be both given or both NULL");
  if (!aligned16(o_ext) || (extra_o && !aligned16(extra_o)))
    return fail(FB_ERR_ALIGN, "o_ext and extra_o must be 16-byte aligned");
  st = check_ws(ws, ws_bytes, workspace_for(d, sp));
  if (st != FB_OK) return st;
  return run_combine(d, sp ? sp->mode : fb::CHUNKS_ALL, sp, extra_o, extra_lse, o_ext, lse_ext, ws, ws_bytes,
                     stream);
}

fb_status fb_block_attn(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk,
                        const float* o_ext, const float* lse_ext, void* o, float* lse_out, void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st == FB_OK) st = check_plans(d, nullptr, false, true);
  if (st != FB_OK) return st;
  if (!q_blk || !k_blk || !v_blk || !o) return fail(FB_ERR_NULL, "q_blk, k_blk, v_blk and o are required");
  if ((o_ext == nullptr) != (lse_ext == nullptr))
    return fail(FB_ERR_NULL, "o_ext and lse_ext must be both given or both NULL");
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o) ||
      (o_ext && !aligned16(o_ext)))
    return fail(FB_ERR_ALIGN, "q_blk, k_blk, v_blk, o and o_ext must be 16-byte aligned");
  return run_block(d, q_blk, k_blk, v_blk, o_ext, lse_ext, o, lse_out, stream);
}

fb_status fb_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a, const float* o_b,
                   const float* lse_b, float* o, float* lse, void* stream) {
  clear_error();
  if (rows < 0 || rows > (1LL << 36)) return fail(FB_ERR_SHAPE, "rows = %lld out of range", (long long)rows);
  if (head_dim < 4 || head_dim > 1024 || head_dim % 4 != 0)
    return fail(FB_ERR_UNSUPPORTED, "head_dim %d must be a multiple of 4 in [4, 1024]", head_dim);
  if (rows == 0) return FB_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return fail(FB_ERR_NULL, "fb_merge: NULL pointer");
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o)) return fail(FB_ERR_ALIGN, "fb_merge: o_a, o_b, o must be 16-byte aligned");
  return hip_status(fb::launch_merge(rows, head_dim, o_a, lse_a, o_b, lse_b, o, lse, stream), "merge launch");
}

}  // extern "C"


// Argument checks of fb_step and fb_step_noalloc (everything but the
// workspace); *need receives the workspace the step uses.
static fb_status step_checks(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk,
                             const void* k_pre, const void* v_pre, const fb_sparse* sp, float* o_ext_cache,
                             float* lse_ext_cache, float* o_res_cache, float* lse_res_cache, void* o, int32_t step,
                             int32_t refresh_period, int32_t mode, size_t* need) {
  fb_status st = check_desc(d);
  if (st == FB_OK) st = check_offsets(d);
  if (st == FB_OK) st = check_sparse(sp, false);
  if (st == FB_OK) st = check_plans(d, sp, true, true);
  if (st != FB_OK) return st;
  if (step < 0) return fail(FB_ERR_ARG, "step = %d < 0", step);
  if (refresh_period < 1) return fail(FB_ERR_ARG, "refresh_period = %d < 1", refresh_period);
  if (mode != FB_MODE_CACHED && mode != FB_MODE_FULL) return fail(FB_ERR_ARG, "mode = %d", mode);
  if (!q_blk || !k_blk || !v_blk || !o_ext_cache || !lse_ext_cache || !o)
    return fail(FB_ERR_NULL, "q_blk, k_blk, v_blk, o_ext_cache, lse_ext_cache and o are required");
  if (total_prefix(d) > 0 && (!k_pre || !v_pre))
    return fail(FB_ERR_NULL, "k_pre and v_pre are required for a non-empty prefix");
  if (sp && (!o_res_cache || !lse_res_cache))
    return fail(FB_ERR_NULL, "the sparse variant needs o_res_cache and lse_res_cache");
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_pre) || !aligned16(v_pre) ||
      !aligned16(o_ext_cache) || !aligned16(o) || (sp && !aligned16(o_res_cache)))
    return fail(FB_ERR_ALIGN, "all tensor base pointers must be 16-byte aligned");
  *need = workspace_for(d, sp);
  return FB_OK;
}

// The step itself, after step_checks and a workspace of at least *need bytes.
static fb_status step_run(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk,
                          const void* k_pre, const void* v_pre, const fb_sparse* sp, float* o_ext_cache,
                          float* lse_ext_cache, float* o_res_cache, float* lse_res_cache, void* o, float* lse_out,
                          int32_t step, int32_t refresh_period, int32_t mode, int32_t force_refresh,
                          int32_t* refreshed_out, void* ws, size_t ws_bytes, void* stream) {
  fb_status st = FB_OK;
  const bool refresh = mode == FB_MODE_FULL || force_refresh != 0 || step % refresh_period == 0;
  st = debug_chunk_check(d, sp, ws, stream);
  if (st != FB_OK) return st;
  if (refreshed_out) *refreshed_out = refresh ? 1 : 0;
  if (!refresh && debug_checks() && !capturing(stream)) {
    // the partial this step reuses: the block-external cache, or the residual in the sparse variant
    const float* oc = sp ? o_res_cache : o_ext_cache;
    const float* lc = sp ? lse_res_cache : lse_ext_cache;
    st = cache_has_nan(d, oc, lc, ws, step, stream);
    if (st != FB_OK) return st;
  }
  if (!sp) {
    if (refresh) {
      st = run_prefix(d, q_blk, k_pre, v_pre, fb::CHUNKS_ALL, nullptr, nullptr, nullptr, o_ext_cache,
                      lse_ext_cache, ws, ws_bytes, stream);
      if (st != FB_OK) return st;
    }
  } else {
    if (refresh) {
      st = run_prefix(d, q_blk, k_pre, v_pre, fb::CHUNKS_COMPLEMENT, sp, nullptr, nullptr, o_res_cache,
                      lse_res_cache, ws, ws_bytes, stream);
      if (st != FB_OK) return st;
    }
    st = run_prefix(d, q_blk, k_pre, v_pre, fb::CHUNKS_SELECTED, sp, o_res_cache, lse_res_cache, o_ext_cache,
                    lse_ext_cache, ws, ws_bytes, stream);
    if (st != FB_OK) return st;
  }
  return run_block(d, q_blk, k_blk, v_blk, o_ext_cache, lse_ext_cache, o, lse_out, stream);
}

extern "C" {

fb_status fb_step(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pre,
                  const void* v_pre, const fb_sparse* sp, float* o_ext_cache, float* lse_ext_cache,
                  float* o_res_cache, float* lse_res_cache, void* o, float* lse_out, int32_t step,
                  int32_t refresh_period, int32_t mode, int32_t force_refresh, int32_t* refreshed_out, void* ws,
                  size_t ws_bytes, void* stream) {
  clear_error();
  size_t need = 0;
  fb_status st = step_checks(d, q_blk, k_blk, v_blk, k_pre, v_pre, sp, o_ext_cache, lse_ext_cache, o_res_cache,
                             lse_res_cache, o, step, refresh_period, mode, &need);
  if (st == FB_OK) st = check_ws(ws, ws_bytes, need);
  if (st != FB_OK) return st;
  return step_run(d, q_blk, k_blk, v_blk, k_pre, v_pre, sp, o_ext_cache, lse_ext_cache, o_res_cache, lse_res_cache,
                  o, lse_out, step, refresh_period, mode, force_refresh, refreshed_out, ws, ws_bytes, stream);
}

fb_status fb_step_noalloc(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk,
                          const void* k_pre, const void* v_pre, const fb_sparse* sp, float* o_ext_cache,
                          float* lse_ext_cache, float* o_res_cache, float* lse_res_cache, void* o, float* lse_out,
                          int32_t step, int32_t refresh_period, int32_t mode, int32_t force_refresh,
                          int32_t* refreshed_out, void* stream) {
  clear_error();
  size_t need = 0;
  fb_status st = step_checks(d, q_blk, k_blk, v_blk, k_pre, v_pre, sp, o_ext_cache, lse_ext_cache, o_res_cache,
                             lse_res_cache, o, step, refresh_period, mode, &need);
  if (st != FB_OK) return st;
  if (need > fb::kNoAllocScratchBytes)
    return fail(FB_ERR_WORKSPACE, "fb_step_noalloc: this shape needs %zu bytes of scratch, more than the %zu "
                "bytes the library holds per GPU (use fb_step with a workspace)", need, fb::kNoAllocScratchBytes);
  void* ws = nullptr;
  st = hip_status(fb::noalloc_scratch(&ws), "fb_step_noalloc scratch address");
  if (st != FB_OK) return st;
  return step_run(d, q_blk, k_blk, v_blk, k_pre, v_pre, sp, o_ext_cache, lse_ext_cache, o_res_cache, lse_res_cache,
                  o, lse_out, step, refresh_period, mode, force_refresh, refreshed_out, ws, fb::kNoAllocScratchBytes,
                  stream);
}

fb_status fb_refresh_mask_tau(const fb_desc* d, const void* k_prev, const void* v_prev, const void* k_cur,
                              const void* v_cur, float eps, int32_t tau, int32_t step, int32_t* count_out,
                              int32_t* mask_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st != FB_OK) return st;
  if (step < 0) return fail(FB_ERR_ARG, "step = %d < 0", step);
  if (!(eps >= 0.f)) return fail(FB_ERR_ARG, "eps must be >= 0");
  if (!count_out || !mask_out) return fail(FB_ERR_NULL, "count_out and mask_out are required");
  if (step > 0 && (!k_prev || !v_prev || !k_cur || !v_cur))
    return fail(FB_ERR_NULL, "k_prev, v_prev, k_cur and v_cur are required after step 0");
  if (step > 0 && (!aligned16(k_prev) || !aligned16(v_prev) || !aligned16(k_cur) || !aligned16(v_cur)))
    return fail(FB_ERR_ALIGN, "k_prev, v_prev, k_cur and v_cur must be 16-byte aligned");
  const size_t need = (size_t)d->batch * d->block_len * sizeof(int32_t);
  if (ws_bytes < need) return fail(FB_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!ws) return fail(FB_ERR_NULL, "workspace is NULL");
  fb::TauArgs t;
  memset(&t, 0, sizeof(t));
  t.k_prev = k_prev;   // not read at step 0, where every token counts as new
  t.v_prev = v_prev;
  t.k_cur = k_cur;
  t.v_cur = v_cur;
  t.kv_sb = d->kv_stride_b;
  t.kv_st = d->kv_stride_t;
  t.kv_sh = d->kv_stride_h;
  t.B = d->batch;
  t.Lb = d->block_len;
  t.Hkv = d->hkv;
  t.D = d->head_dim;
  t.dtype = d->dtype;
  t.eps = eps;
  t.tau = tau;
  t.step = step;
  t.flags = (int32_t*)ws;
  t.count = count_out;
  t.mask = mask_out;
  return hip_status(fb::launch_tau(t, stream), "tau mask launch");
}

fb_status fb_refresh_mask_gamma(const fb_desc* d, const void* q_cur, void* q_ref, float gamma, int32_t step,
                                float* sim_out, int32_t* mask_out, void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st != FB_OK) return st;
  if (step < 0) return fail(FB_ERR_ARG, "step = %d < 0", step);
  if (gamma != gamma) return fail(FB_ERR_ARG, "gamma is NaN");
  if (!q_cur || !q_ref || !sim_out || !mask_out)
    return fail(FB_ERR_NULL, "q_cur, q_ref, sim_out and mask_out are required");
  if (!aligned16(q_cur) || !aligned16(q_ref)) return fail(FB_ERR_ALIGN, "q_cur and q_ref must be 16-byte aligned");
  fb::GammaArgs g;
  memset(&g, 0, sizeof(g));
  g.q_cur = q_cur;
  g.q_sb = d->q_stride_b;
  g.q_st = d->q_stride_t;
  g.q_sh = d->q_stride_h;
  g.q_ref = q_ref;
  g.B = d->batch;
  g.Lb = d->block_len;
  g.Hq = d->hq;
  g.Hkv = d->hkv;
  g.D = d->head_dim;
  g.dtype = d->dtype;
  g.gamma = gamma;
  g.step = step;
  g.sim = sim_out;
  g.mask = mask_out;
  return hip_status(fb::launch_gamma(g, stream), "gamma mask launch");
}

fb_status fb_step_masked(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk,
                         const void* k_pre, const void* v_pre, const int32_t* mask, float* o_ext_cache,
                         float* lse_ext_cache, void* o, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st == FB_OK) st = check_offsets(d);
  if (st == FB_OK) st = check_plans(d, nullptr, true, true);
  if (st != FB_OK) return st;
  if (!q_blk || !k_blk || !v_blk || !mask || !o_ext_cache || !lse_ext_cache || !o)
    return fail(FB_ERR_NULL, "q_blk, k_blk, v_blk, mask, o_ext_cache, lse_ext_cache and o are required");
  if (total_prefix(d) > 0 && (!k_pre || !v_pre))
    return fail(FB_ERR_NULL, "k_pre and v_pre are required for a non-empty prefix");
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_pre) || !aligned16(v_pre) ||
      !aligned16(o_ext_cache) || !aligned16(o))
    return fail(FB_ERR_ALIGN, "all tensor base pointers must be 16-byte aligned");
  st = check_ws(ws, ws_bytes, workspace_for(d, nullptr));
  if (st != FB_OK) return st;
  // the unit plan of the pairs the mask recomputes, after the partials
  PrefixPlan p;
  st = plan_prefix(d, fb::CHUNKS_ALL, 0, 64, &p);
  if (st != FB_OK) return st;
  fb::UnitPlanArgs u;
  memset(&u, 0, sizeof(u));
  u.mask = mask;
  u.offsets = d->prefix_offsets_dev;
  u.B = d->batch;
  u.Hkv = d->hkv;
  u.row_tiles = p.row_tiles;
  u.min_split = d->dtype == FB_F32 ? 1 : kMinSplitTiles;
  u.cap = p.n_work;
  u.plan = (int32_t*)((char*)ws + p.part_o_bytes + p.part_lse_bytes);
  st = hip_status(fb::launch_unit_plan(u, stream), "unit plan launch");
  if (st != FB_OK) return st;
  st = run_prefix(d, q_blk, k_pre, v_pre, fb::CHUNKS_ALL, nullptr, nullptr, nullptr, o_ext_cache, lse_ext_cache,
                  ws, ws_bytes, stream, u.plan);
  if (st != FB_OK) return st;
  return run_block(d, q_blk, k_blk, v_blk, o_ext_cache, lse_ext_cache, o, lse_out, stream);
}

fb_status fb_append_block(const fb_desc* d, const void* k_blk, const void* v_blk, void* k_pre, void* v_pre,
                          const int64_t* dst_rows_dev, void* stream) {
  clear_error();
  fb_status st = check_desc(d);
  if (st != FB_OK) return st;
  if (!k_blk || !v_blk || !k_pre || !v_pre || !dst_rows_dev)
    return fail(FB_ERR_NULL, "k_blk, v_blk, k_pre, v_pre and dst_rows_dev are required");
  if (!aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_pre) || !aligned16(v_pre))
    return fail(FB_ERR_ALIGN, "all tensor base pointers must be 16-byte aligned");
  if ((int64_t)d->batch * d->block_len * d->hkv * d->head_dim > (1LL << 40))
    return fail(FB_ERR_SHAPE, "block too large");
  fb::AppendArgs a;
  memset(&a, 0, sizeof(a));
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.k_pre = k_pre;
  a.v_pre = v_pre;
  a.kv_sb = d->kv_stride_b;
  a.kv_st = d->kv_stride_t;
  a.kv_sh = d->kv_stride_h;
  a.pre_st = d->pre_stride_t;
  a.pre_sh = d->pre_stride_h;
  a.dst_rows = dst_rows_dev;
  a.B = d->batch;
  a.Lb = d->block_len;
  a.Hkv = d->hkv;
  a.D = d->head_dim;
  a.esize = esize(d);
  return hip_status(fb::launch_append(a, stream), "block append launch");
}

}  // extern "C"

// Chunk counts of the streams: n_max (and n_min) of ceil(Lp_b / chunk_len).
static fb_status chunk_geometry(const fb_desc* d, int32_t chunk_len, int32_t* n_max, int32_t* n_min) {
  fb_status st = check_desc(d);
  if (st == FB_OK) st = check_offsets(d);
  if (st != FB_OK) return st;
  if (chunk_len < 1) return fail(FB_ERR_ARG, "chunk_len = %d < 1", chunk_len);
  int64_t hi = 0, lo = INT64_MAX;
  for (int b = 0; b < d->batch; ++b) {
    const int64_t n = ceil_div(d->prefix_offsets_host[b + 1] - d->prefix_offsets_host[b], chunk_len);
    hi = std::max(hi, n);
    lo = std::min(lo, n);
  }
  // the scoring grid has one workgroup per 64 chunks of every (stream, KV head)
  if (hi * d->batch * d->hkv > (1LL << 26)) return fail(FB_ERR_SHAPE, "too many chunks");
  *n_max = (int32_t)hi;
  *n_min = (int32_t)lo;
  return FB_OK;
}

static void fill_select(fb::SelectArgs& a, const fb_desc* d, int32_t chunk_len, int32_t chunk_cap, int32_t n_max) {
  memset(&a, 0, sizeof(a));
  a.q_sb = d->q_stride_b;
  a.q_st = d->q_stride_t;
  a.q_sh = d->q_stride_h;
  a.pre_st = d->pre_stride_t;
  a.pre_sh = d->pre_stride_h;
  a.offsets = d->prefix_offsets_dev;
  a.B = d->batch;
  a.Hq = d->hq;
  a.Hkv = d->hkv;
  a.G = d->hq / d->hkv;
  a.Lb = d->block_len;
  a.D = d->head_dim;
  a.dtype = d->dtype;
  a.chunk_len = chunk_len;
  a.chunk_cap = chunk_cap;
  a.max_chunks = n_max;
}

static fb_status select_checks(const fb_desc* d, int32_t k, int32_t n_max, int32_t n_min, const void* q_blk,
                               const void* idx) {
  if (k < 1) return fail(FB_ERR_ARG, "k = %d < 1", k);
  if (n_min < k) return fail(FB_ERR_ARG, "a stream has %d chunks < k = %d", n_min, k);
  if (n_max > fb::kMaxSelectChunks) return fail(FB_ERR_SHAPE, "a stream has %d chunks > %d", n_max, fb::kMaxSelectChunks);
  if (!q_blk || !idx) return fail(FB_ERR_NULL, "q_blk and chunk_idx_out are required");
  if (!aligned16(q_blk)) return fail(FB_ERR_ALIGN, "q_blk must be 16-byte aligned");
  (void)d;
  return FB_OK;
}

static size_t pooled_bytes(const fb_desc* d, int32_t cap) {
  return align_up((size_t)d->batch * cap * d->hkv * d->head_dim * sizeof(float));
}

extern "C" {

size_t fb_select_chunks_ws(const fb_desc* d, int32_t chunk_len) {
  clear_error();
  int32_t n_max = 0, n_min = 0;
  if (chunk_geometry(d, chunk_len, &n_max, &n_min) != FB_OK) return 0;
  const size_t scores = align_up((size_t)d->batch * d->hkv * n_max * sizeof(float));
  return std::max<size_t>(pooled_bytes(d, n_max) + scores, kAlign);
}

fb_status fb_pool_chunk_keys(const fb_desc* d, const void* k_pre, int32_t chunk_len, int32_t chunk_cap,
                             int32_t first_chunk, float* pooled, void* stream) {
  clear_error();
  int32_t n_max = 0, n_min = 0;
  fb_status st = chunk_geometry(d, chunk_len, &n_max, &n_min);
  if (st != FB_OK) return st;
  if (chunk_cap < n_max) return fail(FB_ERR_ARG, "chunk_cap = %d < %d chunks of the longest stream", chunk_cap, n_max);
  if (first_chunk < 0) return fail(FB_ERR_ARG, "first_chunk = %d < 0", first_chunk);
  if (!k_pre || !pooled) return fail(FB_ERR_NULL, "k_pre and pooled are required");
  if (!aligned16(k_pre) || !aligned16(pooled)) return fail(FB_ERR_ALIGN, "k_pre and pooled must be 16-byte aligned");
  if (first_chunk >= n_max) return FB_OK;
  fb::SelectArgs a;
  fill_select(a, d, chunk_len, chunk_cap, n_max);
  a.k_pre = k_pre;
  a.first_chunk = first_chunk;
  a.pooled = pooled;
  return hip_status(fb::launch_pool(a, stream), "chunk pooling launch");
}

fb_status fb_select_chunks_pooled(const fb_desc* d, const void* q_blk, const float* pooled, int32_t chunk_len,
                                  int32_t chunk_cap, int32_t k, float* scores, int32_t* chunk_idx_out,
                                  void* stream) {
  clear_error();
  int32_t n_max = 0, n_min = 0;
  fb_status st = chunk_geometry(d, chunk_len, &n_max, &n_min);
  if (st == FB_OK) st = select_checks(d, k, n_max, n_min, q_blk, chunk_idx_out);
  if (st != FB_OK) return st;
  if (chunk_cap < n_max) return fail(FB_ERR_ARG, "chunk_cap = %d < %d chunks of the longest stream", chunk_cap, n_max);
  if (!pooled || !scores) return fail(FB_ERR_NULL, "pooled and scores are required");
  if (!aligned16(pooled)) return fail(FB_ERR_ALIGN, "pooled must be 16-byte aligned");
  fb::SelectArgs a;
  fill_select(a, d, chunk_len, chunk_cap, n_max);
  a.q = q_blk;
  a.k = k;
  a.pooled = (float*)pooled;
  a.scores = scores;
  a.idx_out = chunk_idx_out;
  return hip_status(fb::launch_select_pooled(a, stream), "chunk selection launch");
}

fb_status fb_select_chunks(const fb_desc* d, const void* q_blk, const void* k_pre, int32_t chunk_len, int32_t k,
                           int32_t* chunk_idx_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int32_t n_max = 0, n_min = 0;
  fb_status st = chunk_geometry(d, chunk_len, &n_max, &n_min);
  if (st == FB_OK) st = select_checks(d, k, n_max, n_min, q_blk, chunk_idx_out);
  if (st != FB_OK) return st;
  if (!k_pre) return fail(FB_ERR_NULL, "k_pre is required");
  if (!aligned16(k_pre)) return fail(FB_ERR_ALIGN, "k_pre must be 16-byte aligned");
  const size_t need = fb_select_chunks_ws(d, chunk_len);
  st = check_ws(ws, ws_bytes, need);
  if (st != FB_OK) return st;
  fb::SelectArgs a;
  fill_select(a, d, chunk_len, n_max, n_max);
  a.q = q_blk;
  a.k_pre = k_pre;
  a.k = k;
  a.pooled = (float*)ws;
  a.scores = (float*)((char*)ws + pooled_bytes(d, n_max));
  a.idx_out = chunk_idx_out;
  int rc = fb::launch_pool(a, stream);
  if (rc == 0) rc = fb::launch_select_pooled(a, stream);
  return hip_status(rc, "chunk selection launch");
}

}  // extern "C"
