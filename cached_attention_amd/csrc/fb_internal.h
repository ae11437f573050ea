// Internal launch arguments shared by the host planner (fb_api.cpp) and the
// kernels (fb_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stdint.h>

namespace fb {

enum ChunkMode : int32_t { CHUNKS_ALL = 0, CHUNKS_SELECTED = 1, CHUNKS_COMPLEMENT = 2 };

constexpr int kTile = 64;  // keys per LDS tile

// One attention pass: rows of query heads over a key range, either the packed
// ragged prefix (offsets != nullptr; split over tiles) or each stream's own
// block (offsets == nullptr; one split per stream covering its Lb keys).
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
};

// launchers (fb_kernels.hip); return hipError_t as int
int launch_attn(const AttnArgs& a, int dtype, int head_dim, int qt, bool partial, void* stream);
int launch_combine(const CombineArgs& c, int64_t rows, void* stream);
int launch_merge(int64_t rows, int32_t head_dim, const float* oa, const float* la, const float* ob,
                 const float* lb, float* o, float* lse, void* stream);

}  // namespace fb
