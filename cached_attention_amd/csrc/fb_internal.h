// Internal launch arguments shared by the host planner (fb_api.cpp) and the
// kernels (fb_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace fb {

enum ChunkMode : int32_t { CHUNKS_ALL = 0, CHUNKS_SELECTED = 1, CHUNKS_COMPLEMENT = 2 };

constexpr int kTile = 64;  // keys per LDS tile
constexpr int kDtypeBf16 = 1;  // FB_BF16 of the public header

// bf16 kernel configurations (every one keeps its LDS ring within 64 KB at
// head_dim 128: rings that placed direct-to-LDS loads at 64 KB and above
// faulted on MI355X).  X(id, rows per wave / 16, waves, LDS stages,
// resident workgroups per CU, pass: 1 = split partial of the prefix pass,
// 0 = block pass with merge, row waves: the first this many waves hold query
// rows, the others only issue their share of the tile loads, key groups:
// 1, or 2 = the row waves form two groups over the same rows, each taking
// one 32-key half of every tile, merged through LDS at the end).  Query rows
// per workgroup = row waves / key groups * 16 * (rows per wave / 16).
#define FB_BF16_CFGS(X)                                                \
  X(4, 1, 4, 2, 2, 0, 4, 1)      /* block   64 rows                          */ \
  X(5, 1, 8, 2, 1, 0, 8, 1)      /* block  128 rows                          */ \
  X(7, 2, 4, 2, 2, 1, 4, 1)      /* prefix 128 rows, 2 workgroups per CU     */ \
  X(9, 1, 2, 2, 2, 1, 2, 1)      /* prefix  32 rows, 2 workgroups per CU     */ \
  X(10, 1, 4, 2, 2, 1, 4, 1)     /* prefix  64 rows, 2 workgroups per CU     */ \
  X(18, 2, 8, 2, 1, 0, 8, 1)     /* block  256 rows: 8 waves x 32            */ \
  X(19, 2, 4, 2, 2, 0, 4, 1)     /* block  128 rows, 2 workgroups per CU     */ \
  X(21, 1, 2, 2, 2, 0, 2, 1)     /* block   32 rows: 2 waves x 16            */ \
  X(22, 1, 4, 2, 2, 0, 2, 1)     /* block   32 rows + 2 loading waves        */ \
  X(26, 1, 4, 2, 2, 0, 1, 1)     /* block   16 rows + 3 loading waves        */ \
  X(27, 2, 8, 2, 1, 1, 8, 1)     /* prefix 256 rows: 8 waves x 32            */ \
  X(29, 2, 4, 2, 2, 0, 4, 2)     /* block   64 rows: 2 x 32 rows x 2 key halves */ \
  X(30, 1, 10, 2, 1, 0, 10, 2)   /* block   80 rows: 5 x 16 rows x 2 key halves */

enum KernelCfg : int32_t {
  CFG_B64 = 4,
  CFG_B128 = 5,
  CFG_P128_X2 = 7,
  CFG_P32_X2 = 9,
  CFG_P64_X2 = 10,
  CFG_B256 = 18,
  CFG_B128_X2 = 19,
  CFG_B32 = 21,
  CFG_B32_LD = 22,
  CFG_B16_LD = 26,
  CFG_P256 = 27,
  CFG_B64_K2 = 29,
  CFG_B80_K2 = 30,
};

struct CfgInfo {
  int rows;         // query rows per workgroup
  int wgs_per_cu;   // resident workgroups per CU (LDS / register bound)
};
inline CfgInfo cfg_info(int cfg) {
  switch (cfg) {
#define FB_CFG_INFO(ID, QT, NW, NS, WPC, PART, RW, KG) \
    case ID: return {(RW) / (KG) * 16 * (QT), WPC};
    FB_BF16_CFGS(FB_CFG_INFO)
#undef FB_CFG_INFO
    default: return {64, 1};
  }
}

struct AttnArgs {
  // queries [B][Lb][Hq][D] with element strides
  const void* q;
  int64_t q_sb, q_st, q_sh;
  int32_t B, Hq, Hkv, G, Lb, rows;  // rows = G * Lb query rows per KV head
  float c_log2;                     // softmax scale * log2(e)
  // keys / values
  const void* k;
  const void* v;
  int64_t kv_sb, kv_st, kv_sh;
  const int64_t* offsets;  // device prefix offsets [B+1], or nullptr for block keys
  // work decomposition
  int32_t split_tiles;     // logical tiles per split
  int32_t row_tiles;       // row tiles per KV head
  int32_t n_work;          // real workgroups
  int32_t grid;            // launched workgroups (multiple of 8)
  // sparse chunk list [B][Hkv][n_sel]
  const int32_t* chunks;
  int32_t n_sel, chunk_tiles, chunk_mode;
  // partial outputs [split][Hq][Lb][D], [split][Hq][Lb]
  float* part_o;
  float* part_lse;
  // merged output: cache partial to merge with (nullable), o [B][Lb][Hq][D], lse [B][Hq][Lb]
  const float* ext_o;
  const float* ext_lse;
  void* o;
  float* lse_out;
  // unit plan of a masked step (nullable = every (stream, KV head)): the
  // workgroups map onto the listed (stream, KV head) pairs only, and the
  // partials are packed per listed pair (layout below)
  const int32_t* plan;
};

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  const int64_t* offsets;
  int32_t B, Hq, Lb, D;
  int32_t split_tiles, n_sel, chunk_tiles, chunk_mode;
  int32_t total_splits;    // partials in the workspace (split indices are clamped to it)
  const float* extra_o;    // optional extra partial [B][Hq][Lb][D] folded in (sparse residual)
  const float* extra_lse;
  float* o;                // [B][Hq][Lb][D]
  float* lse;              // [B][Hq][Lb]
  const int32_t* plan;     // unit plan (nullable = every head): rows of unlisted heads are left untouched
  int32_t Hkv, G;
  int32_t max_splits;      // most splits of any stream (without a unit plan; the plan's are unknown on the host)
};
constexpr int kFewSplits = 4;   // rows of at most this many splits take the one-round-trip combine

// Unit plan of a masked step, int32 in device memory, written by
// launch_unit_plan from a [B][Hkv] recompute mask (P = B * Hkv pairs):
//   [0] workgroups with work (units * row tiles)   [1] tiles per split
//   [2] listed pairs n                              [3] units (splits of all listed pairs)
//   [4 .. 4+P)       pair b * Hkv + g of listed pair a (a < n), in mask order
//   [4+P .. 5+2P)    first unit of listed pair a (a <= n; [n] = units)
//   [5+2P .. 5+3P)   listed index of pair b * Hkv + g, or -1
// Unit u holds G * Lb partial rows (query head of the group, block position).
inline int64_t plan_ints(int64_t pairs) { return 5 + 3 * pairs; }
struct UnitPlanArgs {
  const int32_t* mask;      // [B][Hkv], nonzero = recompute
  const int64_t* offsets;   // device prefix offsets [B+1]
  int32_t B, Hkv, row_tiles, min_split;
  int32_t cap;              // at most this many workgroups (the all-heads plan's)
  int32_t* plan;
};
int launch_unit_plan(const UnitPlanArgs& u, void* stream);

// Adaptive reuse masks.
struct TauArgs {
  const void* k_prev;
  const void* v_prev;
  const void* k_cur;
  const void* v_cur;
  int64_t kv_sb, kv_st, kv_sh;
  int32_t B, Lb, Hkv, D, dtype;
  float eps;
  int32_t tau, step;
  int32_t* flags;    // [B][Lb] scratch
  int32_t* count;    // [B]
  int32_t* mask;     // [B][Hkv]
};
struct GammaArgs {
  const void* q_cur;
  int64_t q_sb, q_st, q_sh;
  void* q_ref;       // [B][Lb][Hq][D] contiguous, same dtype
  int32_t B, Lb, Hq, Hkv, D, dtype;
  float gamma;
  int32_t step;
  float* sim;        // [B][Hq]
  int32_t* mask;     // [B][Hkv]
};

// launchers (fb_kernels.hip); return hipError_t as int
int launch_attn(const AttnArgs& a, int dtype, int head_dim, int cfg, bool partial, void* stream);
int launch_combine(const CombineArgs& c, int64_t rows, void* stream);
int launch_merge(int64_t rows, int32_t head_dim, const float* oa, const float* la, const float* ob,
                 const float* lb, float* o, float* lse, void* stream);
int launch_tau(const TauArgs& t, void* stream);
// block append: copy [B][Lb][Hkv][D] rows (block strides) into prefix rows
struct AppendArgs {
  const void* k_blk;
  const void* v_blk;
  void* k_pre;
  void* v_pre;
  int64_t kv_sb, kv_st, kv_sh;   // block strides (elements)
  int64_t pre_st, pre_sh;        // prefix strides (elements)
  const int64_t* dst_rows;       // [B] device
  int32_t B, Lb, Hkv, D, esize;
};
int launch_append(const AppendArgs& a, void* stream);
// chunk selection for the sparse variant: pooled chunk keys, max query score, top-k
constexpr int kMaxSelectChunks = 16384;   // chunks per stream the top-k pass holds in LDS
struct SelectArgs {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const void* k_pre;
  int64_t pre_st, pre_sh;
  const int64_t* offsets;   // device [B+1]
  int32_t B, Hq, Hkv, G, Lb, D, dtype, chunk_len, k;
  int32_t chunk_cap;        // chunk capacity per stream of pooled / scores
  int32_t max_chunks;       // max over streams of ceil(Lp_b / chunk_len)
  int32_t first_chunk;      // pooling: chunks first_chunk .. of every stream
  float* pooled;            // [B][chunk_cap][Hkv][D]
  float* scores;            // [B][Hkv][chunk_cap]
  int32_t* idx_out;         // [B][Hkv][k]
};
int launch_pool(const SelectArgs& a, void* stream);
int launch_select_pooled(const SelectArgs& a, void* stream);
int launch_gamma(const GammaArgs& g, void* stream);
// *flag = 1 if any of x[0..n) is NaN (flag cleared first when clear is set)
int launch_nan_scan(const float* x, int64_t n, int32_t* flag, bool clear, void* stream);
// *flag = 1 unless every [B][Hkv][k] chunk list is strictly ascending and in
// range for its stream (flag cleared first)
int launch_chunk_check(const int32_t* list, const int64_t* offsets, int32_t B, int32_t Hkv, int32_t k,
                       int32_t chunk_len, int32_t* flag, void* stream);

// Scratch of the no-allocation step: a file-scope device array of this many
// bytes in fb_kernels.hip, one per GPU.  *ptr receives its address on the
// calling thread's current device (looked up once per device, thread-safe).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
int noalloc_scratch(void** ptr);

}  // namespace fb
