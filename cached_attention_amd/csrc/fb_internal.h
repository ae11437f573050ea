// Internal launch arguments shared by the host planner (fb_api.cpp) and the
// kernels (fb_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stdint.h>

namespace fb {

enum ChunkMode : int32_t { CHUNKS_ALL = 0, CHUNKS_SELECTED = 1, CHUNKS_COMPLEMENT = 2 };

constexpr int kTile = 64;  // keys per LDS tile
constexpr int kDtypeBf16 = 1;  // FB_BF16 of the public header

// bf16 kernel configurations.  X(id, rows per wave / 16, waves, LDS stages,
// resident workgroups per CU, pass: 1 = split partial of the prefix pass,
// 0 = block pass with merge, row waves: the first this many waves hold query
// rows, the others only issue their share of the tile loads).  Query rows
// per workgroup = row waves * 16 * (rows per wave / 16).
#define FB_BF16_CFGS(X)                                                \
  X(0, 1, 2, 4, 1, 1, 2)      /* prefix  32 rows: 2 waves x 16            */ \
  X(1, 1, 4, 4, 1, 1, 4)      /* prefix  64 rows: 4 waves x 16            */ \
  X(2, 2, 4, 4, 1, 1, 4)      /* prefix 128 rows: 4 waves x 32            */ \
  X(3, 2, 8, 4, 1, 1, 8)      /* prefix 256 rows: 8 waves x 32            */ \
  X(4, 1, 4, 2, 2, 0, 4)      /* block   64 rows                          */ \
  X(5, 1, 8, 2, 1, 0, 8)      /* block  128 rows                          */ \
  X(7, 2, 4, 2, 2, 1, 4)      /* prefix 128 rows, 2 workgroups per CU     */ \
  X(8, 4, 4, 4, 1, 1, 4)      /* prefix 256 rows: 4 waves x 64            */ \
  X(9, 1, 2, 2, 2, 1, 2)      /* prefix  32 rows, 2 workgroups per CU     */ \
  X(10, 1, 4, 2, 2, 1, 4)     /* prefix  64 rows, 2 workgroups per CU     */ \
  X(12, 1, 8, 4, 1, 1, 8)     /* prefix 128 rows: 8 waves x 16            */ \
  X(18, 2, 8, 2, 1, 0, 8)     /* block  256 rows: 8 waves x 32            */ \
  X(19, 2, 4, 2, 2, 0, 4)     /* block  128 rows, 2 workgroups per CU     */ \
  X(20, 4, 4, 4, 1, 0, 4)     /* block  256 rows: 4 waves x 64            */ \
  X(21, 1, 2, 2, 2, 0, 2)     /* block   32 rows: 2 waves x 16            */ \
  X(22, 1, 4, 2, 2, 0, 2)     /* block   32 rows + 2 loading waves        */ \
  X(26, 1, 4, 2, 2, 0, 1)     /* block   16 rows + 3 loading waves        */

enum KernelCfg : int32_t {
  CFG_P32 = 0,
  CFG_P64 = 1,
  CFG_P128 = 2,
  CFG_P256 = 3,
  CFG_B64 = 4,
  CFG_B128 = 5,
  CFG_P128_X2 = 7,
  CFG_P256_Q4 = 8,
  CFG_P32_X2 = 9,
  CFG_P64_X2 = 10,
  CFG_P128_W8 = 12,
  CFG_B256 = 18,
  CFG_B128_X2 = 19,
  CFG_B256_Q4 = 20,
  CFG_B32 = 21,
  CFG_B32_LD = 22,
  CFG_B16_LD = 26,
};

struct CfgInfo {
  int rows;         // query rows per workgroup
  int wgs_per_cu;   // resident workgroups per CU (LDS / register bound)
};
inline CfgInfo cfg_info(int cfg) {
  switch (cfg) {
#define FB_CFG_INFO(ID, QT, NW, NS, WPC, PART, RW) \
    case ID: return {(RW) * 16 * (QT), WPC};
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
  // per-(stream, KV head) recompute mask [B][Hkv] (nullable = all): workgroups
  // of a masked-out head exit at once
  const int32_t* head_mask;
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
  const int32_t* head_mask;  // [B][Hkv] (nullable = all): rows of masked-out heads are left untouched
  int32_t Hkv, G;
};

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

}  // namespace fb
