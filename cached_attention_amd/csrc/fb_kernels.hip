// HIP kernels of the FlashBlock attention step for gfx950 (MI355X).
//
// attn_bf16  -- attention of a workgroup's query rows over one key range,
//              bf16 in, fp32 accumulate on MFMA.  Used twice:
//                * prefix pass (block-external partial A_out, L_out = log Z_out
//                  of the FlashBlock "Core Mechanism" section): split-KV over
//                  the packed ragged prefix, writes fp32 partials per split;
//                * block pass (block-internal partial A_in, bidirectional):
//                  one split per stream over its Lb block keys, merged in
//                  registers with the cached (A_out, L_out) by the page's merge
//                  equation and written in bf16.
// attn_f32   -- the same two passes in plain fp32 VALU arithmetic.
// combine    -- log-sum-exp combination of the split partials (the merge
//              equation generalised to n partials), optionally folding in one
//              more partial (the sparse variant's cached residual).
// merge      -- the merge equation on two fp32 partials.
//
// Layout of one bf16 LDS stage (64 keys, head_dim D):
//   K tile  [64 keys][D]   row = 2D bytes, 16-byte slot c of key t stored at
//                          slot c ^ (t & 7)
//   V^T tile [D][64 keys]  row = 128 bytes; keys stored in the order in which
//                          the score MFMA leaves P in registers, 16-byte slot s
//                          of row d stored at s ^ ((d ^ (d >> 3)) & 7)
// The XOR swizzles keep the 16-byte LDS reads of the MFMA operands and the
// 16-byte writes of the staging threads free of bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fb_internal.h"

namespace fb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// ---------------------------------------------------------------------------
// Split plan, evaluated identically by the attention and combine kernels.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int64_t prefix_len(const int64_t* off, int b) { return off[b + 1] - off[b]; }

// Logical tiles of stream b: SELECTED walks the listed chunks, otherwise the
// prefix positions (COMPLEMENT skips listed chunks while walking).
__device__ __forceinline__ int logical_tiles(const int64_t* off, int b, int chunk_mode, int n_sel,
                                             int chunk_tiles) {
  if (chunk_mode == CHUNKS_SELECTED) return n_sel * chunk_tiles;
  return (int)((prefix_len(off, b) + kTile - 1) / kTile);
}

__device__ __forceinline__ int splits_of(const int64_t* off, int b, int split_tiles, int chunk_mode,
                                         int n_sel, int chunk_tiles) {
  int n = logical_tiles(off, b, chunk_mode, n_sel, chunk_tiles);
  return (n + split_tiles - 1) / split_tiles;
}

// ---------------------------------------------------------------------------
// Tile iterator over one split (wave-uniform state).
// ---------------------------------------------------------------------------

struct TileIter {
  int lt, lt_end;
  int64_t lp;
  const int32_t* list;
  int nlist, ptr, mode, ct;
};

__device__ __forceinline__ bool next_tile(TileIter& it, int64_t& tok0, int& nvalid) {
  while (it.lt < it.lt_end) {
    const int i = it.lt++;
    int64_t start;
    if (it.mode == CHUNKS_SELECTED) {
      const int64_t c = it.list[i / it.ct];
      start = (c * it.ct + (i % it.ct)) * (int64_t)kTile;
      if (c < 0 || start >= it.lp) continue;
    } else {
      start = (int64_t)i * kTile;
      if (it.mode == CHUNKS_COMPLEMENT) {
        const int c = i / it.ct;
        while (it.ptr < it.nlist && it.list[it.ptr] < c) ++it.ptr;
        if (it.ptr < it.nlist && it.list[it.ptr] == c) continue;
      }
    }
    tok0 = start;
    const int64_t rem = it.lp - start;
    nvalid = rem < kTile ? (int)rem : kTile;
    return true;
  }
  return false;
}

// Decodes workgroup -> (split x, KV head g, row tile rt) with an XCD-aware
// remap: consecutive workgroup ids go round-robin over the 8 XCDs, so ids
// L, L+8, L+16, ... share an XCD; they get consecutive work items, which puts
// the row tiles of one (split, KV head) -- readers of the same keys -- on one
// XCD's L2.  Then finds the stream b and the logical-tile range of the split.
struct Work {
  int x, g, rt, b;
  TileIter it;
  const char* kbase;
  const char* vbase;
};

template <int ESZ>
__device__ __forceinline__ bool decode_work(const AttnArgs& a, Work& wk) {
  const int L = blockIdx.x;
  const int per = a.grid >> 3;
  const int w = (L & 7) * per + (L >> 3);
  if (w >= a.n_work) return false;
  wk.rt = w % a.row_tiles;
  const int gx = w / a.row_tiles;
  wk.g = gx % a.Hkv;
  wk.x = gx / a.Hkv;
  TileIter& it = wk.it;
  it.list = nullptr;
  it.nlist = 0;
  it.ptr = 0;
  it.mode = CHUNKS_ALL;
  it.ct = 1;
  int64_t tok_base;
  if (a.offsets) {
    int acc = 0, b = 0, j = 0;
    for (; b < a.B; ++b) {
      const int ns = splits_of(a.offsets, b, a.split_tiles, a.chunk_mode, a.n_sel, a.chunk_tiles);
      if (wk.x < acc + ns) {
        j = wk.x - acc;
        break;
      }
      acc += ns;
    }
    if (b >= a.B) return false;
    wk.b = b;
    it.lp = prefix_len(a.offsets, b);
    const int nl = logical_tiles(a.offsets, b, a.chunk_mode, a.n_sel, a.chunk_tiles);
    it.lt = j * a.split_tiles;
    it.lt_end = min(nl, it.lt + a.split_tiles);
    it.mode = a.chunk_mode;
    if (a.chunk_mode != CHUNKS_ALL) {
      it.list = a.chunks + ((int64_t)b * a.Hkv + wk.g) * a.n_sel;
      it.nlist = a.n_sel;
      it.ct = a.chunk_tiles;
      if (a.chunk_mode == CHUNKS_COMPLEMENT) {  // first listed chunk >= first chunk of the split
        const int c0 = it.lt / it.ct;
        int lo = 0, hi = it.nlist;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (it.list[mid] < c0) lo = mid + 1; else hi = mid;
        }
        it.ptr = lo;
      }
    }
    tok_base = a.offsets[b];
    wk.kbase = (const char*)a.k + (tok_base * a.kv_st + (int64_t)wk.g * a.kv_sh) * ESZ;
    wk.vbase = (const char*)a.v + (tok_base * a.kv_st + (int64_t)wk.g * a.kv_sh) * ESZ;
  } else {
    wk.b = wk.x;
    it.lp = a.Lb;
    it.lt = 0;
    it.lt_end = (a.Lb + kTile - 1) / kTile;
    wk.kbase = (const char*)a.k + ((int64_t)wk.b * a.kv_sb + (int64_t)wk.g * a.kv_sh) * ESZ;
    wk.vbase = (const char*)a.v + ((int64_t)wk.b * a.kv_sb + (int64_t)wk.g * a.kv_sh) * ESZ;
  }
  return true;
}

// ---------------------------------------------------------------------------
// bf16 attention on MFMA
// ---------------------------------------------------------------------------
//
// Workgroup: 4 waves; wave w owns 16*QT consecutive query rows of one KV head
// (row i -> query head g*G + i / Lb, block position i % Lb).  Per 64-key tile:
//   S^T[key][q] = K Q^T      v_mfma_f32_16x16x32_bf16, A = K from LDS,
//                            B = Q^T held in VGPRs for the whole pass
//   online softmax on S^T    each lane holds one query column (lane & 15) and
//                            16 keys of it; row max over the 4 lane groups by
//                            two xor-shuffles; exp2 with scale*log2(e) folded in
//   O^T[d][q] += V^T P^T     A = V^T from LDS, B = P^T straight from the score
//                            accumulators (bf16), no cross-lane movement
// Staging: 256 units of eight 16-byte global loads per tile (half K, half V),
// loaded into VGPRs one tile ahead and written to the other LDS stage after
// the current tile's MFMAs; V is transposed in registers (8x8 bf16 blocks).

template <int D, int QT, bool PARTIAL>
__global__ void __launch_bounds__(256) attn_bf16(const AttnArgs a) {
  constexpr int KS = D / 32;            // k-steps of the score MFMA
  constexpr int DT = D / 16;            // 16-row d tiles of O^T
  constexpr int CH = D / 8;             // 16-byte chunks per key row
  constexpr int ROWS = 64 * QT;         // query rows per workgroup
  constexpr int KBYTES = kTile * D * 2;
  constexpr int STAGE = 2 * KBYTES;
  constexpr int HALF_UNITS = (kTile / 8) * CH;  // K units == V units
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  Work wk;
  if (!decode_work<2>(a, wk)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // ---- query fragments (B operand of the score MFMA) ----
  const int row_w0 = wk.rt * ROWS + wave * 16 * QT;
  const bool wave_active = row_w0 < a.rows;
  bf16x8 qf[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = row_w0 + qt * 16 + l16;
    if (row < a.rows) {
      const int h = wk.g * a.G + row / a.Lb;
      const int pos = row % a.Lb;
      const __bf16* qp = (const __bf16*)a.q + (int64_t)wk.b * a.q_sb + (int64_t)pos * a.q_st +
                         (int64_t)h * a.q_sh + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qt][ks] = *(const bf16x8*)(qp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qt][ks] = (bf16x8){};
    }
  }

  f32x4 oacc[DT][QT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = kNegInf;
    l_run[qt] = 0.f;
  }

  // ---- staging role of this thread ----
  const bool is_k = tid < HALF_UNITS;
  const bool is_v = !is_k && tid < 2 * HALF_UNITS;
  const int unit = is_k ? tid : tid - HALF_UNITS;
  const int uc = unit % CH;   // 16-byte chunk (8 dims)
  const int ug = unit / CH;   // group of 8 keys
  int utok[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (is_k) {
      utok[r] = ug * 8 + r;
    } else {  // keys whose P values one lane group holds for one 32-key MFMA step
      const int jj = ug >> 2, gq = ug & 3;
      utok[r] = jj * 32 + (r < 4 ? 4 * gq + r : 16 + 4 * gq + (r - 4));
    }
  }
  const char* gsrc = is_k ? wk.kbase : wk.vbase;
  const int64_t row_bytes = a.kv_st * 2;
  u32x4 stg[8];

  auto stage_load = [&](int64_t tok0, int nvalid) {
    if (!(is_k || is_v)) return;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (utok[r] < nvalid)
        stg[r] = *(const u32x4*)(gsrc + (tok0 + utok[r]) * row_bytes + uc * 16);
      else
        stg[r] = (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto stage_store = [&](int buf) {
    char* base = smem + buf * STAGE;
    if (is_k) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        *(u32x4*)(base + (ug * 8 + r) * (D * 2) + ((uc ^ r) * 16)) = stg[r];
    } else if (is_v) {
      const int slot = ((ug >> 2) << 2) | (ug & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = uc * 8 + e;
        const int dw = e >> 1;
        u32x4 outv;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t x0 = stg[2 * kk][dw];
          const uint32_t x1 = stg[2 * kk + 1][dw];
          outv[kk] = (e & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
        }
        const int phys = slot ^ ((d ^ (d >> 3)) & 7);
        *(u32x4*)(base + KBYTES + d * 128 + phys * 16) = outv;
      }
    }
  };

  const float c = a.c_log2;

  auto compute = [&](int buf, int nvalid) {
    const char* Ks = smem + buf * STAGE;
    const char* Vs = Ks + KBYTES;
    f32x4 s[4][QT];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = tt * 16 + l16;
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int slot = ks * 4 + lg;
        kf[ks] = *(const bf16x8*)(Ks + tok * (D * 2) + ((slot ^ (tok & 7)) * 16));
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[qt][ks], acc, 0, 0, 0);
        s[tt][qt] = acc;
      }
    }
    if (nvalid < kTile) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = tt * 16 + 4 * lg + i >= nvalid;
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            if (dead) s[tt][qt][i] = kNegInf;
        }
    }
    bf16x8 pf[2][QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = kNegInf;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][qt][i]);
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float m_new = fmaxf(m_run[qt], mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
      m_run[qt] = m_new;
      float rs = 0.f;
      uint32_t pk[4][2];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][qt][i], c, -m_new));
          rs += p[i];
        }
        pk[tt][0] = pack_bf16x2(p[0], p[1]);
        pk[tt][1] = pack_bf16x2(p[2], p[3]);
      }
      l_run[qt] = l_run[qt] * alpha + rs;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        u32x4 pv = {pk[2 * jj][0], pk[2 * jj][1], pk[2 * jj + 1][0], pk[2 * jj + 1][1]};
        pf[jj][qt] = __builtin_bit_cast(bf16x8, pv);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 16 + l16;
        const int slot = jj * 4 + lg;
        const bf16x8 vf = *(const bf16x8*)(Vs + d * 128 + ((slot ^ ((d ^ (d >> 3)) & 7)) * 16));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[jj][qt], oacc[dt][qt], 0, 0, 0);
      }
    }
  };

  // ---- pipelined main loop: global loads of tile i+1 overlap compute of tile i ----
  int64_t tok_cur = 0, tok_nxt = 0;
  int nv_cur = 0, nv_nxt = 0;
  bool have_cur = next_tile(wk.it, tok_cur, nv_cur);
  if (have_cur) {
    stage_load(tok_cur, nv_cur);
    stage_store(0);
  }
  __syncthreads();
  bool have_nxt = have_cur && next_tile(wk.it, tok_nxt, nv_nxt);
  int buf = 0;
  while (have_cur) {
    if (have_nxt) stage_load(tok_nxt, nv_nxt);
    if (wave_active) compute(buf, nv_cur);
    if (have_nxt) stage_store(buf ^ 1);
    __syncthreads();
    have_cur = have_nxt;
    tok_cur = tok_nxt;
    nv_cur = nv_nxt;
    buf ^= 1;
    if (have_cur) have_nxt = next_tile(wk.it, tok_nxt, nv_nxt);
  }

  if (!wave_active) return;

  // ---- epilogue ----
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float lt = l_run[qt];
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    const int row = row_w0 + qt * 16 + l16;
    if (row >= a.rows) continue;
    const int h = wk.g * a.G + row / a.Lb;
    const int pos = row % a.Lb;
    const bool any = lt > 0.f;
    const float inv = any ? 1.f / lt : 0.f;
    const float lse = any ? (m_run[qt] + __log2f(lt)) * kLn2 : kNegInf;
    if constexpr (PARTIAL) {
      const int64_t prow = ((int64_t)wk.x * a.Hq + h) * a.Lb + pos;
      float* po = a.part_o + prow * D + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4*)(po + dt * 16) = oacc[dt][qt] * inv;
      if (lg == 0) a.part_lse[prow] = lse;
    } else {
      const int64_t crow = ((int64_t)wk.b * a.Hq + h) * a.Lb + pos;
      const float le = a.ext_lse ? a.ext_lse[crow] : kNegInf;
      const float mm = fmaxf(le, lse);
      const float we = __expf(le - mm);
      const float wi = __expf(lse - mm);
      const float den = we + wi;
      const float rden = 1.f / den;
      const float wi_n = wi * inv * rden;
      const float we_n = we * rden;
      __bf16* op = (__bf16*)a.o + (((int64_t)wk.b * a.Lb + pos) * a.Hq + h) * D + 4 * lg;
      const float* ep = a.ext_o ? a.ext_o + crow * D + 4 * lg : nullptr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 r = oacc[dt][qt] * wi_n;
        if (ep) r += *(const f32x4*)(ep + dt * 16) * we_n;
        u32x2 packed = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        *(u32x2*)(op + dt * 16) = packed;
      }
      if (lg == 0 && a.lse_out) a.lse_out[crow] = mm + __logf(den);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 attention (plain VALU): one wave per workgroup, one query row per lane
// ---------------------------------------------------------------------------

template <int D, bool PARTIAL>
__global__ void __launch_bounds__(64) attn_f32(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float Kt[kTile][D];
  __shared__ __attribute__((aligned(16))) float Vt[kTile][D];
  Work wk;
  if (!decode_work<4>(a, wk)) return;
  const int lane = threadIdx.x;
  const int row = wk.rt * 64 + lane;
  const bool active = row < a.rows;
  int h = 0, pos = 0;
  float q[D], acc[D];
  if (active) {
    h = wk.g * a.G + row / a.Lb;
    pos = row % a.Lb;
    const float* qp = (const float*)a.q + (int64_t)wk.b * a.q_sb + (int64_t)pos * a.q_st + (int64_t)h * a.q_sh;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const f32x4 v = *(const f32x4*)(qp + d);
      q[d] = v[0]; q[d + 1] = v[1]; q[d + 2] = v[2]; q[d + 3] = v[3];
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const float c = a.c_log2;
  const int64_t row_bytes = a.kv_st * 4;
  int64_t tok0;
  int nvalid;
  while (next_tile(wk.it, tok0, nvalid)) {
    __syncthreads();
    for (int idx = lane; idx < kTile * (D / 4); idx += 64) {
      const int t = idx / (D / 4), ch = idx % (D / 4);
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (t < nvalid) {
        kv = *(const f32x4*)(wk.kbase + (tok0 + t) * row_bytes + ch * 16);
        vv = *(const f32x4*)(wk.vbase + (tok0 + t) * row_bytes + ch * 16);
      }
      *(f32x4*)&Kt[t][ch * 4] = kv;
      *(f32x4*)&Vt[t][ch * 4] = vv;
    }
    __syncthreads();
    if (!active) continue;
    for (int t = 0; t < nvalid; ++t) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], Kt[t][d], s);
      const float ts = s * c;
      const float m_new = fmaxf(m_run, ts);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      const float p = __builtin_amdgcn_exp2f(ts - m_new);
      m_run = m_new;
      l_run = l_run * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, Vt[t][d], acc[d] * alpha);
    }
  }
  if (!active) return;
  const bool any = l_run > 0.f;
  const float inv = any ? 1.f / l_run : 0.f;
  const float lse = any ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
  if constexpr (PARTIAL) {
    const int64_t prow = ((int64_t)wk.x * a.Hq + h) * a.Lb + pos;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int d = 0; d < D; ++d) po[d] = acc[d] * inv;
    a.part_lse[prow] = lse;
  } else {
    const int64_t crow = ((int64_t)wk.b * a.Hq + h) * a.Lb + pos;
    const float le = a.ext_lse ? a.ext_lse[crow] : kNegInf;
    const float mm = fmaxf(le, lse);
    const float we = expf(le - mm);
    const float wi = expf(lse - mm);
    const float den = we + wi;
    float* op = (float*)a.o + (((int64_t)wk.b * a.Lb + pos) * a.Hq + h) * D;
    const float* ep = a.ext_o ? a.ext_o + crow * D : nullptr;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      float r = wi * acc[d] * inv;
      if (ep) r += we * ep[d];
      op[d] = r / den;
    }
    if (a.lse_out) a.lse_out[crow] = mm + logf(den);
  }
}

// ---------------------------------------------------------------------------
// split combine: one wave per (stream, head, block position) row
// ---------------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs c, int64_t rows) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t hl = (int64_t)c.Hq * c.Lb;
  const int b = (int)(row / hl);
  const int64_t rem = row % hl;
  int x0 = 0;
  for (int bb = 0; bb < b; ++bb) x0 += splits_of(c.offsets, bb, c.split_tiles, c.chunk_mode, c.n_sel, c.chunk_tiles);
  int ns = splits_of(c.offsets, b, c.split_tiles, c.chunk_mode, c.n_sel, c.chunk_tiles);
  if (x0 > c.total_splits) x0 = c.total_splits;
  if (ns > c.total_splits - x0) ns = c.total_splits - x0;
  float mx = kNegInf;
  for (int x = x0; x < x0 + ns; ++x) mx = fmaxf(mx, c.part_lse[(int64_t)x * hl + rem]);
  const float le = c.extra_lse ? c.extra_lse[row] : kNegInf;
  mx = fmaxf(mx, le);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (mx != kNegInf) {
    for (int x = x0; x < x0 + ns; ++x) {
      const int64_t pr = (int64_t)x * hl + rem;
      const float w = expf(c.part_lse[pr] - mx);
      wsum += w;
      const float* po = c.part_o + pr * D + lane * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(w, po[i], acc[i]);
    }
    if (c.extra_lse) {
      const float w = expf(le - mx);
      wsum += w;
      const float* po = c.extra_o + row * D + lane * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(w, po[i], acc[i]);
    }
  }
  const bool any = wsum > 0.f;
  const float inv = any ? 1.f / wsum : 0.f;
  float* op = c.o + row * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) op[i] = acc[i] * inv;
  if (lane == 0) c.lse[row] = any ? mx + logf(wsum) : kNegInf;
}

// ---------------------------------------------------------------------------
// two-partial merge: one wave per row (all reads of a row precede its writes)
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) merge_kernel(int64_t rows, int D, const float* oa, const float* la,
                                                    const float* ob, const float* lb, float* o, float* lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float l1 = la[row], l2 = lb[row];
  const float mm = fmaxf(l1, l2);
  const bool empty = mm == kNegInf;
  const float w1 = empty ? 0.f : expf(l1 - mm);
  const float w2 = empty ? 0.f : expf(l2 - mm);
  const float den = w1 + w2;
  const float inv = empty ? 0.f : 1.f / den;
  // each lane reads its own 16-byte chunks and writes them back in place, so
  // o may alias oa or ob; lse is written after every lane has read la / lb
  for (int ch = lane; ch < D / 4; ch += 64) {
    const f32x4 a4 = *(const f32x4*)(oa + row * D + ch * 4);
    const f32x4 b4 = *(const f32x4*)(ob + row * D + ch * 4);
    *(f32x4*)(o + row * D + ch * 4) = (a4 * w1 + b4 * w2) * inv;
  }
  if (lane == 0) lse[row] = empty ? kNegInf : mm + logf(den);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int D, int QT, bool P>
static int launch_bf16(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16<D, QT, P>), dim3(a.grid), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

template <int D, bool P>
static int launch_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_f32<D, P>), dim3(a.grid), dim3(64), 0, s, a);
  return (int)hipGetLastError();
}

int launch_attn(const AttnArgs& a, int dtype, int head_dim, int qt, bool partial, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.grid == 0) return 0;
  if (dtype == 0) {  // fp32
    if (head_dim == 64) return partial ? launch_f32<64, true>(a, s) : launch_f32<64, false>(a, s);
    return partial ? launch_f32<128, true>(a, s) : launch_f32<128, false>(a, s);
  }
#define FB_DISPATCH_QT(DD)                                                             \
  switch (qt) {                                                                        \
    case 1: return partial ? launch_bf16<DD, 1, true>(a, s) : launch_bf16<DD, 1, false>(a, s); \
    case 2: return partial ? launch_bf16<DD, 2, true>(a, s) : launch_bf16<DD, 2, false>(a, s); \
    default: return partial ? launch_bf16<DD, 4, true>(a, s) : launch_bf16<DD, 4, false>(a, s); \
  }
  if (head_dim == 64) {
    FB_DISPATCH_QT(64)
  }
  FB_DISPATCH_QT(128)
#undef FB_DISPATCH_QT
}

int launch_combine(const CombineArgs& c, int64_t rows, void* stream) {
  if (rows == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (c.D == 64)
    hipLaunchKernelGGL((combine_kernel<64>), grid, dim3(256), 0, s, c, rows);
  else
    hipLaunchKernelGGL((combine_kernel<128>), grid, dim3(256), 0, s, c, rows);
  return (int)hipGetLastError();
}

int launch_merge(int64_t rows, int32_t head_dim, const float* oa, const float* la, const float* ob,
                 const float* lb, float* o, float* lse, void* stream) {
  if (rows == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, rows, head_dim, oa, la,
                     ob, lb, o, lse);
  return (int)hipGetLastError();
}

}  // namespace fb
