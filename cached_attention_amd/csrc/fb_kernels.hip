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
// attn_f32m  -- the same two passes in fp32 on v_mfma_f32_16x16x4_f32.
// combine    -- log-sum-exp combination of the split partials (the merge
//              equation generalised to n partials), optionally folding in one
//              more partial (the sparse variant's cached residual).
// merge      -- the merge equation on two fp32 partials.
// tau_flags / tau_finalize, gamma
//            -- the adaptive reuse decisions: updated-token counts and
//              per-head query similarities, turned into recompute masks.
// append     -- the finalised block's K/V rows into the prefix cache.
// pool / score / topk
//            -- chunk selection for the sparse variant: mean-pooled chunk
//              keys, max query score per chunk, top-k by radix select.
// flag_clear / nan_scan / chunk_check
//            -- the opt-in debug checks (a cache before a reuse step, a
//              sparse chunk list).
// unit_plan  -- the device work list of a masked step: the recomputed
//              (stream, KV head) pairs and their split length.
// scratch    -- the per-GPU device array of the no-allocation step.
//
// Layout of one bf16 LDS stage (64 keys, head_dim D): the K tile, then the V
// tile, each row-major [64 keys][D] (row = 2D bytes) as the direct-to-LDS
// loads write them.  Both use one XOR swizzle of 16-byte slots: slot c of key
// t is stored at c ^ 2*(t & 7) (D = 128; c ^ 2*(t & 3) at D = 64), even
// values only, so the two slots of one 16-dim column block stay adjacent for
// the transpose reads.  K fragments are read with 16-byte LDS reads, V^T
// fragments with ds_read_b64_tr_b16; the counters read no bank conflicts.
// Block passes of 1024 rows and more per KV head split every tile between two
// key groups of waves (keys 0..31 and 32..63); after the last tile the ring
// holds group 1's (O, m, l) for group 0 to merge.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

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

// Read-only kernel inputs (offsets, chunk lists) are read through the constant
// address space: wave-uniform loads then become scalar loads, which do not
// count against vmcnt and so never stall the direct-to-LDS pipeline.
#define FB_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const FB_CONST T*)p)[i];
}

// ---------------------------------------------------------------------------
// Split plan, evaluated identically by the attention and combine kernels.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int64_t prefix_len(const int64_t* off, int b) {
  return ld_const(off, b + 1) - ld_const(off, b);
}

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
  int lt, lt_end, step;   // logical tiles lt, lt + step, ... below lt_end (step > 1: interleaved splits)
  int64_t lp;
  const int32_t* list;
  int nlist, ptr, mode, ct;
};

// DENSE: the caller knows the iterator walks every position (no chunk list),
// so the chunk-mode code is left out of its tile loop
template <bool DENSE = false>
__device__ __forceinline__ bool next_tile(TileIter& it, int64_t& tok0, int& nvalid) {
  if (DENSE || it.mode == CHUNKS_ALL) {   // wave-uniform: one scalar branch per tile
    if (it.lt >= it.lt_end) return false;
    const int64_t start = (int64_t)it.lt * kTile;
    it.lt += it.step;
    tok0 = start;
    const int64_t rem = it.lp - start;
    nvalid = rem < kTile ? (int)rem : kTile;
    return true;
  }
  while (it.lt < it.lt_end) {
    const int i = it.lt++;
    int64_t start;
    if (it.mode == CHUNKS_SELECTED) {
      const int64_t c = ld_const(it.list, i / it.ct);
      start = (c * it.ct + (i % it.ct)) * (int64_t)kTile;
      if (c < 0 || start >= it.lp) continue;
    } else {
      start = (int64_t)i * kTile;
      if (it.mode == CHUNKS_COMPLEMENT) {
        const int c = i / it.ct;
        while (it.ptr < it.nlist && ld_const(it.list, it.ptr) < c) ++it.ptr;
        if (it.ptr < it.nlist && ld_const(it.list, it.ptr) == c) continue;
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
  int hs, h_off;   // partial row of query head h: (x * hs + h_off + h - g * G) * Lb + position
  TileIter it;
  const char* kbase;
  const char* vbase;
};

template <int ESZ, bool INTERLEAVE = false>
__device__ __forceinline__ bool decode_work(const AttnArgs& a, Work& wk) {
  const int L = blockIdx.x;
  const int per = a.grid >> 3;
  const int w = (L & 7) * per + (L >> 3);
  TileIter& it = wk.it;
  it.step = 1;
  it.list = nullptr;
  it.nlist = 0;
  it.ptr = 0;
  it.mode = CHUNKS_ALL;
  it.ct = 1;
  int64_t tok_base;
  wk.hs = a.Hq;
  if (a.offsets && a.plan) {
    // masked step: unit u = w / row_tiles is split j of the listed pair that
    // holds it (the last pair whose first unit is <= u)
    const int32_t* pl = a.plan;
    if (w >= ld_const(pl, 0)) return false;
    const int st = ld_const(pl, 1), n = ld_const(pl, 2);
    const int P = a.B * a.Hkv;
    const int32_t* base = pl + 4 + P;
    wk.rt = w % a.row_tiles;
    const int u = w / a.row_tiles;
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ld_const(base, mid) <= u) lo = mid; else hi = mid - 1;
    }
    const int bg = ld_const(pl + 4, lo);
    wk.b = bg / a.Hkv;
    wk.g = bg % a.Hkv;
    wk.x = u;
    wk.hs = a.G;   // units hold only their group's query heads
    wk.h_off = 0;
    const int j = u - ld_const(base, lo);
    it.lp = prefix_len(a.offsets, wk.b);
    const int nl = (int)((it.lp + kTile - 1) / kTile);
    it.lt = j * st;
    it.lt_end = min(nl, it.lt + st);
    tok_base = ld_const(a.offsets, wk.b);
    wk.kbase = (const char*)a.k + (tok_base * a.kv_st + (int64_t)wk.g * a.kv_sh) * ESZ;
    wk.vbase = (const char*)a.v + (tok_base * a.kv_st + (int64_t)wk.g * a.kv_sh) * ESZ;
    return true;
  }
  if (w >= a.n_work) return false;
  wk.rt = w % a.row_tiles;
  const int gx = w / a.row_tiles;
  wk.g = gx % a.Hkv;
  wk.x = gx / a.Hkv;
  wk.h_off = wk.g * a.G;
  if (a.offsets) {
    int acc = 0, b = 0, j = 0, nsb = 0;
    for (; b < a.B; ++b) {
      const int ns = splits_of(a.offsets, b, a.split_tiles, a.chunk_mode, a.n_sel, a.chunk_tiles);
      if (wk.x < acc + ns) {
        j = wk.x - acc;
        nsb = ns;
        break;
      }
      acc += ns;
    }
    if (b >= a.B) return false;
    wk.b = b;
    it.lp = prefix_len(a.offsets, b);
    const int nl = logical_tiles(a.offsets, b, a.chunk_mode, a.n_sel, a.chunk_tiles);
    if (INTERLEAVE && a.chunk_mode == CHUNKS_ALL) {
      // split j of the stream's nsb takes tiles j, j + nsb, j + 2 nsb, ...:
      // at most split_tiles of them, and the splits of a KV head read
      // neighbouring tiles at the same time
      it.lt = j;
      it.lt_end = nl;
      it.step = nsb;
    } else {
      it.lt = j * a.split_tiles;
      it.lt_end = min(nl, it.lt + a.split_tiles);
    }
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
          if (ld_const(it.list, mid) < c0) lo = mid + 1; else hi = mid;
        }
        it.ptr = lo;
      }
    }
    tok_base = ld_const(a.offsets, b);
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
// Workgroup: NW waves; wave w < RW owns 16*QT consecutive query rows of one KV
// head (row i -> query head g*G + i / Lb, block position i % Lb); waves RW ..
// NW-1 hold no rows and only issue their share of the tile loads.  With KG = 2
// key groups (block pass only) waves w and w + NW/2 own the same rows, the
// first taking keys 0..31 of every tile and the second keys 32..63; each
// group keeps its own softmax reference, and the two partials are merged
// through LDS before the epilogue.  Per 64-key tile (per 32-key half):
//   S^T[key][q] = K Q^T      v_mfma_f32_16x16x32_bf16, A = K from LDS,
//                            B = Q^T held in VGPRs for the whole pass
//   online softmax on S^T    each lane holds one query column (lane & 15) and
//                            16 keys of it; row max over the 4 lane groups by
//                            two xor-shuffles; exp2 with scale*log2(e) folded in
//   O^T[d][q] += V^T P^T     A = V^T read from the row-major V tile with the
//                            LDS transpose read, B = P^T straight from the
//                            score accumulators (bf16), no cross-lane movement
// Keys and values move HBM -> LDS with direct-to-LDS loads into an NS-stage
// ring, DIST tiles ahead of the tile being computed; each wave waits only for
// the tile it is about to read (per-stage vmcnt), then one barrier per tile.
//
// LDS operands are read ahead into registers: the K fragments of k-step
// ks+1 while the MFMAs of step ks run, and the V^T fragments kVAhead MFMA
// groups ahead of their use (the first ones before the softmax, whose VALU
// work covers their latency).
//
// Softmax reference: each pass (one split of the prefix, or the block) runs
// against a fixed per-row reference m, the exact row maxima of its first tile
// (peeled out of the tile loop); every later tile computes p = exp2(s*c - m)
// with no max reduction, no rescale of O and no per-tile check.  Row sums
// accumulate the bf16-rounded p that the PV product uses (v_dot2), so O and l
// are normalised consistently.  After the last tile each row's l bounds all of
// its p: if some l exceeds 2^80 (or is infinite) a score outran the reference
// by more than about 55 nats within the split -- rare -- and the workgroup
// finds the split's exact row maxima with a scores-only pass and runs the pass
// again against them, where no p exceeds 1.  The normalised result does not
// depend on the reference.

constexpr float kSumLimit = 1.2089258e24f;   // 2^80: a row sum beyond it sends the pass to the rerun

#define FB_LDS __attribute__((address_space(3)))

template <int N>
struct IC {
  static constexpr int value = N;
};

// s_waitcnt vmcnt(n) for n = k * per, k in [0, 3] (gfx9 encoding: expcnt and
// lgkmcnt left at their maxima)
template <int PER>
__device__ __forceinline__ void wait_vmcnt_tiles(int k) {
  constexpr int base = 0x0F70;
  switch (k) {
    case 0: __builtin_amdgcn_s_waitcnt(base | 0); break;
    case 1: __builtin_amdgcn_s_waitcnt(base | ((PER & 15) | ((PER >> 4) << 14))); break;
    case 2: __builtin_amdgcn_s_waitcnt(base | (((2 * PER) & 15) | (((2 * PER) >> 4) << 14))); break;
    default: __builtin_amdgcn_s_waitcnt(base | (((3 * PER) & 15) | (((3 * PER) >> 4) << 14))); break;
  }
}

// The barrier that precedes a stage's refill.  Each wave first drains its own
// LDS reads (lgkmcnt(0)): the V^T fragments of the deferred PV groups are read
// from the stage the next direct-to-LDS loads overwrite, and nothing else
// orders those reads before another wave's refill.
__device__ __forceinline__ void lds_dma_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__device__ __forceinline__ int kv_swz(int key) {
  // 16-byte slot XOR: even values only, so the two 16-byte slots holding one
  // 16-dim column block stay adjacent (the transpose read fetches 8-byte
  // halves of both)
  return D == 128 ? ((key & 7) << 1) : ((key & 3) << 1);
}

// One direct-to-LDS load: 64 lanes x 16 bytes from sbase + voff[lane] into
// LDS at lds (M0), one contiguous 1 KB block.  Written as asm so that the
// compiler, which cannot tell these asynchronous LDS writes apart from the
// operand reads of other stages, does not drain every load in flight before
// each LDS read; completion is tracked explicitly with per-stage vmcnt waits.
// The instruction has no register outputs.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const void* sbase) {
  // both operands are wave-uniform by construction; readfirstlane makes that
  // explicit so they live in SGPRs
  // (readfirstlane returns a signed int: widen through uint32_t, never by
  // sign extension, or a low word with bit 31 set corrupts the high word)
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane(lds);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t bs = ((uint64_t)b_hi << 32) | (uint64_t)b_lo;
  // M0 (the LDS destination) is an explicit operand, so the compiler knows
  // the asm sets it and keeps no live value of its own there
  asm volatile(
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(bs), "{m0}"(l)
      : "memory");
}

#ifndef FB_V_AHEAD
#define FB_V_AHEAD 2
#endif
#ifndef FB_K_AHEAD
#define FB_K_AHEAD 1
#endif
#ifndef FB_V_AHEAD_Q1
#define FB_V_AHEAD_Q1 FB_V_AHEAD
#endif
#ifndef FB_K_AHEAD_Q1
#define FB_K_AHEAD_Q1 FB_K_AHEAD
#endif
// V^T fragment groups / K fragment k-steps read ahead of their MFMAs, for
// 32-row waves (QT = 2) and for 16-row waves (QT = 1), whose MFMA groups are
// half as long and cover less of the LDS latency
template <int QT>
constexpr int v_ahead() { return QT == 1 ? FB_V_AHEAD_Q1 : FB_V_AHEAD; }
template <int QT>
constexpr int k_ahead() { return QT == 1 ? FB_K_AHEAD_Q1 : FB_K_AHEAD; }
#ifndef FB_PV_DEFER
#define FB_PV_DEFER 2
#endif
// PV MFMA groups of a tile deferred to the start of the next tile, where they
// run while that tile's first K fragments are read from LDS (the same
// accumulation order, so bitwise the same result).  Measured on MI355X: 2
// groups took 2.7% off the 128K GQA prefix pass and 1.5% off the video one
// with a tile loop that tested the chunk mode and the ragged tail on every
// tile; with the current loop they make no measurable difference (128K GQA
// 143.1 against 143.2 us, video 274.8 against 275.4 without them); 4 or 6
// gained nothing.
constexpr int kPvDefer = FB_PV_DEFER;
#ifndef FB_MFMA_PRIO
#define FB_MFMA_PRIO 1
#endif
// raise the wave's issue priority over its MFMA runs, so the matrix core is
// fed first when the waves sharing a SIMD are in different phases (measured
// on MI355X: without it the 128K GQA prefix pass takes 146.0 instead of
// 143.2 us, the video one 282 instead of 275)
template <int P>
__device__ __forceinline__ void mfma_prio() {
  if constexpr (FB_MFMA_PRIO != 0) __builtin_amdgcn_s_setprio(P);
}

#ifndef FB_INTERLEAVE_P256
#define FB_INTERLEAVE_P256 1
#endif
template <int D, int QT, int NW, int NS, int MINW, bool PARTIAL, int RW, int KG>
__global__ void __launch_bounds__(64 * NW, MINW) attn_bf16(const AttnArgs a) {
  constexpr int KS = D / 32;                  // k-steps of the score MFMA
  constexpr int DT = D / 16;                  // 16-row d tiles of O^T
  constexpr int CH = D / 8;                   // 16-byte slots per key row
  constexpr int RWG = RW / KG;                // row waves per key group
  constexpr int ROWS = RWG * 16 * QT;         // query rows per workgroup
  constexpr int TT = 4 / KG;                  // 16-key groups of a tile each wave takes
  constexpr int PH = TT / 2;                  // 32-key halves of a tile each wave takes
  static_assert(RW >= 1 && RW <= NW, "row waves");
  static_assert(KG == 1 || (KG == 2 && RW == NW && !PARTIAL), "key groups: block pass, every wave a row wave");
  constexpr int kVAhead = v_ahead<QT>();
  constexpr int kKAhead = k_ahead<QT>();
  constexpr int TBYTES = kTile * D * 2;       // one K or V tile
  constexpr int STAGE = 2 * TBYTES;
  constexpr int IPT = TBYTES / 1024;          // 1 KB direct-to-LDS loads per tile and tensor
  constexpr int LW = NW > 8 ? 8 : NW;         // waves that issue the tile loads (the first LW)
  constexpr int IPW = 2 * IPT / LW;           // loads per loading wave per tile
  constexpr int RPI = 1024 / (2 * D);         // key rows per load instruction
  constexpr int DIST = NS - 1;                // prefetch distance in tiles
  constexpr int NG = PH * DT;                 // MFMA groups of the PV product
  static_assert(IPT % IPW == 0 && IPW % 2 == 0, "each wave loads an even run of one tensor");
  static_assert(NS >= 2 && NS <= 4, "2..4 stages");
  // The direct-to-LDS loads address LDS through M0.  Rings reaching 64 KB and
  // above (3 and 4 stages at head_dim 128) faulted the GPU, so the ring, and
  // every load destination, stays below 64 KB.
  static_assert(NS * STAGE <= 65536, "LDS ring within 64 KB");
  static_assert((DIST - 1) * IPW < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

  // interleaved splits for the 256-row split-KV pass (see decode_work)
  constexpr bool kInterleave = FB_INTERLEAVE_P256 != 0 && PARTIAL && QT == 2 && NW == 8 && KG == 1;
  Work wk;
  if (!decode_work<2, kInterleave>(a, wk)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: DMA operands stay scalar
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // key group of the wave (wave-uniform): group kg takes keys kofs .. kofs +
  // 64/KG - 1 of every tile; wr = the wave's row slot within its group
  const int kg = KG == 1 ? 0 : wave / (NW / KG);
  const int wr = wave - kg * (NW / KG);
  const int kofs = kg * (kTile / KG);

  // ---- query fragments (B operand of the score MFMA) ----
  const int row_w0 = wk.rt * ROWS + wr * 16 * QT;
  const bool row_wave = wr < RWG;             // waves RW .. NW-1 only load tiles
  const bool wave_active = row_wave && row_w0 < a.rows;
  bf16x8 qf[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = row_w0 + qt * 16 + l16;
    if (row_wave && row < a.rows) {
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

  // ---- block pass: the cached partial it merges with is read before the
  // tiles, so its latency overlaps the pass instead of following it (the
  // small-block configurations, which are latency-bound: 5.6 -> 4.8 us for a
  // 32-token MHA block; the 8-wave big-block configuration is MFMA-bound and
  // keeps its registers) ----
#ifndef FB_EXT_PREFETCH
#define FB_EXT_PREFETCH 1
#endif
  constexpr bool kPre = !PARTIAL && QT == 1 && NW <= 4 && FB_EXT_PREFETCH;
  f32x4 ext_pre[kPre ? QT : 1][kPre ? DT : 1];
  float le_pre[kPre ? QT : 1];
  if constexpr (kPre) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int row = row_w0 + qt * 16 + l16;
      le_pre[qt] = kNegInf;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ext_pre[qt][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (row_wave && row < a.rows) {
        const int64_t crow = ((int64_t)wk.b * a.Hq + wk.g * a.G + row / a.Lb) * a.Lb + row % a.Lb;
        if (a.ext_lse) le_pre[qt] = a.ext_lse[crow];
        if (a.ext_o) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) ext_pre[qt][dt] = *(const f32x4*)(a.ext_o + crow * D + 4 * lg + dt * 16);
        }
      }
    }
  }

  f32x4 oacc[DT][QT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run[QT], l_run[QT], mx_lane[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = kNegInf;
    l_run[qt] = 0.f;
    mx_lane[qt] = kNegInf;
  }
  __shared__ int wg_redo;   // set by any wave whose scores outran the reference
  if (tid == 0) wg_redo = 0;

  // ---- direct-to-LDS tile loads ----
  // Waves 0..LW/2-1 load K, waves LW/2..LW-1 V (waves past LW, in the
  // workgroups of more than 8 waves, load nothing); wave w's IPW instructions
  // cover the 1 KB chunks jj0 .. jj0+IPW-1 of its tensor's tile (RPI key rows
  // each).  Lane -> (key row, 16-byte slot); the slot swizzle is applied on
  // the global side so each instruction writes one contiguous 1 KB block of
  // LDS.  The per-lane part of the global offset depends only on the chunk
  // parity.
  const bool loader = wave < LW;
  const bool dma_v = wave >= LW / 2;
  const int jj0 = loader ? (dma_v ? wave - LW / 2 : wave) * IPW : 0;
  const char* gsrc = dma_v ? wk.vbase : wk.kbase;
  const uint32_t lds_dst = lds0 + (dma_v ? TBYTES : 0) + jj0 * 1024;
  const int64_t row_bytes = a.kv_st * 2;
  uint32_t lane_part[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = par * RPI + lane / CH;
    lane_part[par] = (uint32_t)(row * row_bytes) + ((lane % CH) ^ kv_swz<D>(row)) * 16;
  }
  auto issue = [&](int stage, int64_t tok0, int nvalid) __attribute__((always_inline)) {
    if (!loader) return;   // wave-uniform
    const char* g = gsrc + tok0 * row_bytes;
    const uint32_t dst = lds_dst + stage * STAGE;
    if (nvalid < kTile) {   // ragged tile: rows past the end re-read the last key (masked later)
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int row = (jj0 + u) * RPI + lane / CH;
        const int srow = row < nvalid ? row : nvalid - 1;
        dma16(dst + u * 1024, (uint32_t)(srow * row_bytes) + ((lane % CH) ^ kv_swz<D>(row)) * 16, g);
      }
    } else {
#pragma unroll
      for (int u = 0; u < IPW; ++u)
        dma16(dst + u * 1024, lane_part[u & 1] + (uint32_t)((jj0 + u - (u & 1)) * RPI * row_bytes), g);
    }
  };

  const float c = a.c_log2;
  // per-lane LDS offsets of the K fragment reads (key 16*tt + l16, 16-byte
  // slot 4*ks + lg, swizzled) and of the V transpose reads (key 4*lg +
  // (l16 >> 2), dims 16*dt + 4*(l16 & 3), swizzled)
  uint32_t koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = (kofs + l16) * (2 * D) + (((ks * 4 + lg) ^ kv_swz<D>(l16)) * 16);
  const uint32_t vlane = (kofs + 4 * lg + (l16 >> 2)) * (2 * D) + 8 * (l16 & 3);
  const int vkx = kv_swz<D>(4 * lg + (l16 >> 2)) >> 1;

  f32x4 s[TT][QT];
  // V^T fragments of the deferred PV groups; their P^T operands stay in pf
  bf16x8 vdef[kPvDefer > 0 ? kPvDefer : 1];
  bf16x8 pf[PH][QT];
  auto run_deferred = [&]() __attribute__((always_inline)) {
    if constexpr (kPvDefer > 0) {
      mfma_prio<1>();
#pragma unroll
      for (int d = 0; d < kPvDefer; ++d) {
        const int g = NG - kPvDefer + d;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[g % DT][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vdef[d], pf[g / DT][qt], oacc[g % DT][qt], 0, 0, 0);
      }
      mfma_prio<0>();
    }
  };

  // S^T = K Q^T for the tile at LDS offset kb; k-step outer so that the
  // 4 x QT accumulators of a step are independent MFMA chains.  The K
  // fragments of step ks+1 are read while the MFMAs of step ks run; the
  // scheduling fences keep the compiler from sinking the reads next to
  // their MFMAs, where each group would wait out the LDS latency.
  bf16x8 kf[KS][TT];   // keys kofs + 16*tt + l16, 16-byte slot 4*ks + lg
  auto kload = [&](uint32_t kb, int ks) __attribute__((always_inline)) {
    const FB_LDS char* kp = (const FB_LDS char*)(uintptr_t)(kb + koff[ks]);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) kf[ks][tt] = *(const FB_LDS bf16x8*)(kp + tt * 16 * 2 * D);
  };
  // the first K reads of a tile, issued as early as possible after its barrier
  auto scores_begin = [&](uint32_t kb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kKAhead; ++ks) kload(kb, ks);
  };
  auto scores = [&](uint32_t kb, auto pend_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[tt][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (decltype(pend_tag)::value != 0) {   // the previous tile's last PV groups cover the K reads
      __builtin_amdgcn_sched_barrier(0);
      run_deferred();
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_prio<1>();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + kKAhead < KS) kload(kb, ks + kKAhead);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[tt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][tt], qf[qt][ks], s[tt][qt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_prio<0>();
  };

  // exact row maxima of the tile (4 lane groups share a query column)
  auto row_max = [&](int qt) __attribute__((always_inline)) {
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][qt][i]);
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    return mx * c;
  };
  // p = exp2(s*c - m) against the reference, packed to bf16 for the PV
  // product; the packed values (this lane's 16 keys of each row) are summed
  // into l with v_dot2 against (1, 1)
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(__bf16)1.f, (__bf16)1.f};
  auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float msub = m_run[qt] == kNegInf ? 0.f : m_run[qt];
      uint32_t pk[TT][2];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][qt][i], c, -msub));
        pk[tt][0] = pack_bf16x2(p[0], p[1]);
        pk[tt][1] = pack_bf16x2(p[2], p[3]);
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[tt][h]), ones2, l_run[qt], false);
#pragma unroll
      for (int jj = 0; jj < PH; ++jj) {
        u32x4 pv = {pk[2 * jj][0], pk[2 * jj][1], pk[2 * jj + 1][0], pk[2 * jj + 1][1]};
        pf[jj][qt] = __builtin_bit_cast(bf16x8, pv);
      }
    }
  };

  // softmax of the scores in s (tile with nvalid keys), then O^T += V^T P^T
  // with V at LDS offset vb.  The PV product runs in NG groups (key half jj,
  // d tile dt), each one V^T fragment (two transpose reads) and QT MFMAs.
  // MODE 1: the pass's first tile, which sets the reference; MODE 0: a later
  // tile; MODE 2: scores only, feeding the lane-local maxima mx_lane (the
  // rerun's first pass).
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  auto softmax_pv = [&](uint32_t vb, int nvalid, auto mode_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    bf16x8 vf[NG > 0 ? NG : 1];
    auto vload = [&](int g) __attribute__((always_inline)) {
      const int jj = g / DT, dt = g % DT;
      const uint32_t va = vb + vlane + 32 * (dt ^ vkx) + jj * 32 * 2 * D;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FB_LDS bf16x4*)(uintptr_t)va);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FB_LDS bf16x4*)(uintptr_t)(va + 16 * 2 * D));
      vf[g] = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    if constexpr (MODE != 2) {
#pragma unroll
      for (int g = 0; g < kVAhead; ++g) vload(g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nvalid < kTile) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = kofs + tt * 16 + 4 * lg + i >= nvalid;
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            if (dead) s[tt][qt][i] = kNegInf;
        }
    }
    if constexpr (MODE == 2) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx_lane[qt] = fmaxf(mx_lane[qt], s[tt][qt][i]);
      return;
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) m_run[qt] = row_max(qt);
    }
    exps();
    mfma_prio<1>();
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + kVAhead < NG) vload(g + kVAhead);
      __builtin_amdgcn_sched_barrier(0);
      if (g >= NG - kPvDefer) {
        vdef[g - (NG - kPvDefer)] = vf[g];   // runs at the start of the next tile (or the pass's end)
      } else {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[g % DT][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[g], pf[g / DT][qt], oacc[g % DT][qt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_prio<0>();
  };

  // ---- pipeline: position j of the queue = tile k + j; stage of tile k = st ----
  bool q_have[4] = {false, false, false, false};
  int64_t q_tok[4] = {0, 0, 0, 0};
  int q_nv[4] = {0, 0, 0, 0};
  int st = 0;
  // one tile: wait for it (tiles issued after it may stay in flight), one
  // barrier (every wave is done with the stage refilled next), issue the tile
  // DIST ahead, compute, advance the queue
  auto tile_step = [&](auto mode_tag, auto pend_tag, auto dense_tag) __attribute__((always_inline)) {
    constexpr bool kDense = decltype(dense_tag)::value != 0 || !PARTIAL;
    int after = 0;
#pragma unroll
    for (int j = 1; j < DIST; ++j) after += q_have[j] ? 1 : 0;
    wait_vmcnt_tiles<IPW>(after);
    lds_dma_barrier();
    const uint32_t kb = lds0 + st * STAGE;
    if (wave_active) scores_begin(kb);   // stage st is read, stage st + DIST filled: independent
    q_have[DIST] = q_have[DIST - 1] && next_tile<kDense>(wk.it, q_tok[DIST], q_nv[DIST]);
    if (q_have[DIST]) issue((st + DIST) % NS, q_tok[DIST], q_nv[DIST]);
    if (wave_active) {
      scores(kb, pend_tag);
      softmax_pv(kb + TBYTES, q_nv[0], mode_tag);
    }
#pragma unroll
    for (int j = 0; j < DIST; ++j) {
      q_have[j] = q_have[j + 1];
      q_tok[j] = q_tok[j + 1];
      q_nv[j] = q_nv[j + 1];
    }
    q_have[DIST] = false;
    st = st + 1 == NS ? 0 : st + 1;
  };
  // one pass over the tiles of the split (its first tile in mode first_tag,
  // the others in mode rest_tag); false if it has none
  // dense_tag 1: the split walks every prefix position (no chunk list), so
  // its tile loop carries no chunk-mode code
  auto run_pass = [&](auto first_tag, auto rest_tag, auto dense_tag) __attribute__((always_inline)) -> bool {
    constexpr bool kDense = decltype(dense_tag)::value != 0 || !PARTIAL;
    st = 0;
#pragma unroll
    for (int j = 0; j < DIST; ++j) {
      q_have[j] = (j == 0 || q_have[j - 1]) && next_tile<kDense>(wk.it, q_tok[j], q_nv[j]);
      if (q_have[j]) issue(j, q_tok[j], q_nv[j]);
    }
    if (!q_have[0]) return false;
    // PV groups deferred by a tile run at the start of the next tile of the
    // same pass, and at the pass's end (scores-only passes defer nothing)
    constexpr bool defer = kPvDefer > 0 && decltype(rest_tag)::value != 2;
    tile_step(first_tag, IC<0>{}, dense_tag);
    while (q_have[0]) tile_step(rest_tag, IC<defer ? 1 : 0>{}, dense_tag);
    if constexpr (defer) {
      if (wave_active) run_deferred();
    }
    return true;
  };
  // ---- software-pipelined split-KV pass for 16-row waves ----
  // A 16-row wave has little independent work per tile: its score MFMAs,
  // softmax and PV MFMAs form one dependency chain, and both waves of a SIMD
  // run the same phase between two barriers.  Here the keys are fetched one
  // tile ahead of the values, so that while tile k's softmax runs on the
  // VALU, the score MFMAs of tile k+1 (whose K is already in LDS) run on the
  // matrix core; then tile k's PV product.  The ring layout is unchanged:
  // K(j) and V(j) live in stage j % 2.  Iteration k, after its barrier:
  //   K waves issue K(k+2) into stage k % 2 (K(k) was read in iteration k-1),
  //   V waves issue V(k+1) into stage (k+1) % 2 (V(k-1) was read in k-1);
  // each wave waits for its own loads before the next barrier, so every tile
  // has one iteration to arrive.  The per-row arithmetic and its order are
  // those of the plain pass, so the results are bitwise the same.
#ifndef FB_PIPE_Q1
#define FB_PIPE_Q1 1
#endif
  // Measured on MI355X: 2.3% faster on the 32K MHA prefix pass (98.4 -> 96.2
  // us), but slower on every block pass (video 33.2 -> 37.3 us, text blocks
  // 4.1 -> 4.6 us), so only split-KV passes take it.
  constexpr bool kPipe = QT == 1 && PARTIAL && FB_PIPE_Q1 != 0;
  auto run_pipe = [&](auto dense_tag) __attribute__((always_inline)) -> bool {
    constexpr bool kDense = decltype(dense_tag)::value != 0 || !PARTIAL;
    int64_t tk0, tk1 = 0, tk2 = 0;
    int nv0, nv1 = 0, nv2 = 0;
    if (!next_tile<kDense>(wk.it, tk0, nv0)) return false;   // uniform over the workgroup
    bool h1 = next_tile<kDense>(wk.it, tk1, nv1);
    issue(0, tk0, nv0);                      // K(0) or V(0)
    if (!dma_v && h1) issue(1, tk1, nv1);    // K(1)
    f32x4 sn[4][QT];                          // scores of tile k+1
    uint32_t pkp[4][QT][2];                   // bf16-packed p of tile k
    bf16x8 vfp[NG];
    auto vload_p = [&](uint32_t vb, int g) __attribute__((always_inline)) {
      const int jj = g / DT, dt = g % DT;
      const uint32_t va = vb + vlane + 32 * (dt ^ vkx) + jj * 32 * 2 * D;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FB_LDS bf16x4*)(uintptr_t)va);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FB_LDS bf16x4*)(uintptr_t)(va + 16 * 2 * D));
      vfp[g] = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto mask_s = [&](int nvalid) __attribute__((always_inline)) {
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
    };
    // exponentials of key group tt of s, packed and summed as in exps()
    auto exp_group = [&](int tt) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float msub = m_run[qt] == kNegInf ? 0.f : m_run[qt];
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][qt][i], c, -msub));
        pkp[tt][qt][0] = pack_bf16x2(p[0], p[1]);
        pkp[tt][qt][1] = pack_bf16x2(p[2], p[3]);
      }
    };
    auto exp_finish = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pkp[tt][qt][h]), ones2, l_run[qt],
                                                        false);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          u32x4 pv = {pkp[2 * jj][qt][0], pkp[2 * jj][qt][1], pkp[2 * jj + 1][qt][0], pkp[2 * jj + 1][qt][1]};
          pf[jj][qt] = __builtin_bit_cast(bf16x8, pv);
        }
      }
    };
    wait_vmcnt_tiles<IPW>(0);
    lds_dma_barrier();
    if (wave_active) {   // scores of tile 0 and the pass's reference
      scores_begin(lds0);
      scores(lds0, IC<0>{});
      mask_s(nv0);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) m_run[qt] = row_max(qt);
    }
    int k = 0;
    for (;;) {
      wait_vmcnt_tiles<IPW>(0);
      lds_dma_barrier();
      bool h2 = false;
      if (h1) h2 = next_tile<kDense>(wk.it, tk2, nv2);
      if (!dma_v) {
        if (h2) issue(k & 1, tk2, nv2);          // K(k+2)
      } else {
        if (h1) issue((k + 1) & 1, tk1, nv1);    // V(k+1)
      }
      if (wave_active) {
        const uint32_t kb1 = lds0 + ((k + 1) & 1) * STAGE;
        const uint32_t vb0 = lds0 + (k & 1) * STAGE + TBYTES;
        mask_s(nv0);
        // score MFMAs of tile k+1 interleaved with the exponentials of tile k
        if (h1) {
#pragma unroll
          for (int ks = 0; ks < kKAhead; ++ks) kload(kb1, ks);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (h1 && ks + kKAhead < KS) kload(kb1, ks + kKAhead);
          if (ks == KS - 1) {
#pragma unroll
            for (int g = 0; g < kVAhead; ++g) vload_p(vb0, g);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (h1) {
            mfma_prio<1>();
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
              for (int qt = 0; qt < QT; ++qt)
                sn[tt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    kf[ks][tt], qf[qt][ks], ks == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : sn[tt][qt], 0, 0, 0);
            mfma_prio<0>();
          }
#pragma unroll
          for (int tt = ks * 4 / KS; tt < (ks + 1) * 4 / KS; ++tt) exp_group(tt);
          __builtin_amdgcn_sched_barrier(0);
        }
        exp_finish();
        // tile k's PV product
        mfma_prio<1>();
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (g + kVAhead < NG) vload_p(vb0, g + kVAhead);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            oacc[g % DT][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfp[g], pf[g / DT][qt], oacc[g % DT][qt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_prio<0>();
        if (h1) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) s[tt][qt] = sn[tt][qt];
        }
      }
      if (!h1) break;   // uniform
      tk0 = tk1;
      nv0 = nv1;
      tk1 = tk2;
      nv1 = nv2;
      h1 = h2;
      ++k;
    }
    return true;
  };
  const TileIter it0 = wk.it;
  // the main pass with its tile loop specialised for dense splits (the
  // prefix pass without a chunk list, and every block pass); the rare
  // rerun passes below take the general loop
  bool ran;
  if constexpr (kPipe) {
    ran = (!PARTIAL || wk.it.mode == CHUNKS_ALL) ? run_pipe(IC<1>{}) : run_pipe(IC<0>{});
  } else {
    ran = (!PARTIAL || wk.it.mode == CHUNKS_ALL) ? run_pass(IC<1>{}, IC<0>{}, IC<1>{})
                                                 : run_pass(IC<1>{}, IC<0>{}, IC<0>{});
  }
  if (ran) {
    // did a score outrun its row's reference?  (l bounds every p of the row)
    bool redo = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) redo |= wave_active && l_run[qt] > kSumLimit;
    if (__any(redo) && lane == 0) wg_redo = 1;
    __syncthreads();
    if (wg_redo) {   // rare: the split's exact row maxima, then the pass again against them
      wk.it = it0;
      run_pass(IC<2>{}, IC<2>{}, IC<0>{});
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float mx = mx_lane[qt];
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        m_run[qt] = mx * c;
        l_run[qt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
      wk.it = it0;
      run_pass(IC<0>{}, IC<0>{}, IC<0>{});
    }
  }

  // ---- two key groups: each group finishes half of the head dims, group kg
  // the d tiles [kg * DT/2, (kg + 1) * DT/2).  Through the (now idle) ring,
  // one query sub-tile at a time, each wave hands the other group's half of
  // its O and its (m, l) to its partner wave; both put the two partials on the
  // larger reference and add them.  The epilogue's reads of the cached
  // partial and writes of O are then spread over every wave. ----
  constexpr int DH = KG == 2 ? DT / 2 : DT;   // d tiles each wave finishes
  if constexpr (KG == 2) {
    static_assert(KG * RWG * DH * 64 * 16 + KG * RWG * 64 * 8 <= NS * STAGE, "merge buffer within the ring");
    f32x4* xo = (f32x4*)smem;                                   // [group][RWG][DH][64 lanes]
    float2* xs = (float2*)(smem + KG * RWG * DH * 64 * 16);     // [group][RWG][64 lanes]: (m, l)
    // the accumulators are indexed with compile-time d tiles only (a
    // run-time index would move them to scratch memory): one instance per
    // key group, chosen by the wave-uniform kg
    auto exchange = [&](int qt, auto own_tag) __attribute__((always_inline)) {
      constexpr int own = decltype(own_tag)::value, oth = 1 - own;
#pragma unroll
      for (int e = 0; e < DH; ++e) xo[((own * RWG + wr) * DH + e) * 64 + lane] = oacc[oth * DH + e][qt];
      xs[(own * RWG + wr) * 64 + lane] = make_float2(m_run[qt], l_run[qt]);
    };
    auto merge_own = [&](int qt, auto own_tag) __attribute__((always_inline)) {
      constexpr int own = decltype(own_tag)::value, oth = 1 - own;
      const float2 ml = xs[(oth * RWG + wr) * 64 + lane];
      const float mm = fmaxf(m_run[qt], ml.x);
      // log2-domain references; a group whose keys all fell past the end
      // (reference -inf, zero sum) gets weight 0
      const float a0 = m_run[qt] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[qt] - mm);
      const float a1 = ml.x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(ml.x - mm);
#pragma unroll
      for (int e = 0; e < DH; ++e)
        oacc[own * DH + e][qt] = oacc[own * DH + e][qt] * a0 + xo[((oth * RWG + wr) * DH + e) * 64 + lane] * a1;
      l_run[qt] = l_run[qt] * a0 + ml.y * a1;
      m_run[qt] = mm;
    };
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      __syncthreads();   // every wave is done with the ring (its last tile, or the previous sub-tile)
      if (wave_active) {
        if (kg == 0) exchange(qt, IC<0>{}); else exchange(qt, IC<1>{});
      }
      __syncthreads();
      if (wave_active) {
        if (kg == 0) merge_own(qt, IC<0>{}); else merge_own(qt, IC<1>{});
      }
    }
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
      const int64_t prow = ((int64_t)wk.x * wk.hs + wk.h_off + row / a.Lb) * a.Lb + pos;
      float* po = a.part_o + prow * D + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4*)(po + dt * 16) = oacc[dt][qt] * inv;
      if (lg == 0) a.part_lse[prow] = lse;
    } else {
      const int64_t crow = ((int64_t)wk.b * a.Hq + h) * a.Lb + pos;
      float le;
      if constexpr (kPre) le = le_pre[qt];
      else le = a.ext_lse ? a.ext_lse[crow] : kNegInf;
      const float mm = fmaxf(le, lse);
      const float we = __expf(le - mm);
      const float wi = __expf(lse - mm);
      const float den = we + wi;
      const float rden = 1.f / den;
      const float wi_n = wi * inv * rden;
      const float we_n = we * rden;
      __bf16* op = (__bf16*)a.o + (((int64_t)wk.b * a.Lb + pos) * a.Hq + h) * D + 4 * lg;
      const float* ep = a.ext_o ? a.ext_o + crow * D + 4 * lg : nullptr;
      // the wave's d tiles: all of them, or its key group's half (compile-time
      // tile indices, one instance per group)
      auto store = [&](auto d0_tag) __attribute__((always_inline)) {
        constexpr int d0 = decltype(d0_tag)::value;
#pragma unroll
        for (int e = 0; e < DH; ++e) {
          const int dt = d0 + e;
          f32x4 r = oacc[dt][qt] * wi_n;
          if constexpr (kPre) {
            r += ext_pre[qt][dt] * we_n;   // zeros when there is no cache
          } else {
            if (ep) r += *(const f32x4*)(ep + dt * 16) * we_n;
          }
          u32x2 packed = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
          *(u32x2*)(op + dt * 16) = packed;
        }
      };
      if (KG == 1 || kg == 0) store(IC<0>{}); else store(IC<DH>{});
      if (lg == 0 && kg == 0 && a.lse_out) a.lse_out[crow] = mm + __logf(den);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 attention on MFMA (v_mfma_f32_16x16x4_f32)
// ---------------------------------------------------------------------------
//
// Workgroup: 4 waves x 16 query rows of one KV head (the 64-row tiles of the
// host plan).  Per 64-key tile, staged in LDS with rows padded by 4 floats:
//   S^T[key][q] = K Q^T    A = K from LDS, B = Q^T held in registers; in
//                          k-step ks lane group lg takes dim lg*(D/4) + ks,
//                          so each lane's K and Q values are contiguous
//   online softmax         each lane holds one query column (l16) and keys
//                          16*tt + 4*lg + r; running row max, O rescaled
//   O^T[d][q] += V^T P^T   k-step (tt, r) takes key 16*tt + 4*lg + r in lane
//                          group lg -- the lane's own p, no cross-lane move;
//                          row m of d-tile dt is dim m*DT + dt, so each
//                          lane's V reads are contiguous
// Products and sums stay in fp32 throughout.
template <int D, bool PARTIAL>
__global__ void __launch_bounds__(256) attn_f32m(const AttnArgs a) {
  constexpr int QQ = D / 4;     // dims per lane group = k-steps of the score MFMA
  constexpr int DT = D / 16;    // d tiles of O^T
  constexpr int LDK = D + 4;    // padded LDS row, floats
  __shared__ __attribute__((aligned(16))) float Ks[kTile * LDK];
  __shared__ __attribute__((aligned(16))) float Vs[kTile * LDK];
  Work wk;
  if (!decode_work<4>(a, wk)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int row = wk.rt * 64 + wave * 16 + l16;   // this lane's query column
  const bool rvalid = row < a.rows;
  const bool wave_active = wk.rt * 64 + wave * 16 < a.rows;
  const int h = rvalid ? wk.g * a.G + row / a.Lb : 0;
  const int pos = rvalid ? row % a.Lb : 0;
  float qv[QQ];
#pragma unroll
  for (int i = 0; i < QQ; ++i) qv[i] = 0.f;
  if (rvalid) {
    const float* qp = (const float*)a.q + (int64_t)wk.b * a.q_sb + (int64_t)pos * a.q_st + (int64_t)h * a.q_sh +
                      lg * QQ;
#pragma unroll
    for (int i = 0; i < QQ; i += 4) {
      const f32x4 v = *(const f32x4*)(qp + i);
      qv[i] = v[0]; qv[i + 1] = v[1]; qv[i + 2] = v[2]; qv[i + 3] = v[3];
    }
  }
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;   // l_run: this lane's keys only, summed over lane groups at the end
  const float c = a.c_log2;
  const int64_t row_bytes = a.kv_st * 4;
  int64_t tok0;
  int nvalid;
  while (next_tile<!PARTIAL>(wk.it, tok0, nvalid)) {
    __syncthreads();   // every wave is done with the previous tile
    for (int idx = tid; idx < kTile * (D / 4); idx += 256) {
      const int t = idx / (D / 4), ch = idx % (D / 4);
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};   // keys past the end: zeros
      if (t < nvalid) {
        kv = *(const f32x4*)(wk.kbase + (tok0 + t) * row_bytes + ch * 16);
        vv = *(const f32x4*)(wk.vbase + (tok0 + t) * row_bytes + ch * 16);
      }
      *(f32x4*)&Ks[t * LDK + ch * 4] = kv;
      *(f32x4*)&Vs[t * LDK + ch * 4] = vv;
    }
    __syncthreads();
    if (!wave_active) continue;
    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const float* kp = &Ks[(16 * tt + l16) * LDK + lg * QQ];
#pragma unroll
      for (int i = 0; i < QQ; i += 4) {
        const f32x4 kk = *(const f32x4*)(kp + i);
#pragma unroll
        for (int u = 0; u < 4; ++u) s[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk[u], qv[i + u], s[tt], 0, 0, 0);
      }
    }
    // online softmax in the log2 domain
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * tt + 4 * lg + r;
        s[tt][r] = key < nvalid ? s[tt][r] * c : kNegInf;
        mx = fmaxf(mx, s[tt][r]);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);   // finite: the tile has a valid key
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run = -inf
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[tt][r] = __builtin_amdgcn_exp2f(s[tt][r] - m_new);
        ps += s[tt][r];
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* vp = &Vs[(16 * tt + 4 * lg + r) * LDK + l16 * DT];
#pragma unroll
        for (int d4 = 0; d4 < DT; d4 += 4) {
          const f32x4 vv = *(const f32x4*)(vp + d4);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            oacc[d4 + u] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[u], s[tt][r], oacc[d4 + u], 0, 0, 0);
        }
      }
  }
  if (!wave_active) return;
  float l = l_run;
  l += shfl_xor_f(l, 16);
  l += shfl_xor_f(l, 32);
  if (!rvalid) return;
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const float lse = any ? (m_run + __log2f(l)) * kLn2 : kNegInf;
  // lane (l16, lg) holds O^T rows 4*lg + i of every d tile: dims (4*lg + i)*DT + dt
  if constexpr (PARTIAL) {
    const int64_t prow = ((int64_t)wk.x * wk.hs + wk.h_off + row / a.Lb) * a.Lb + pos;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) po[(4 * lg + i) * DT + dt] = oacc[dt][i] * inv;
    if (lg == 0) a.part_lse[prow] = lse;
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
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = (4 * lg + i) * DT + dt;
        float r = wi * oacc[dt][i] * inv;
        if (ep) r += we * ep[d];
        op[d] = r / den;
      }
    if (lg == 0 && a.lse_out) a.lse_out[crow] = mm + logf(den);
  }
}

// ---------------------------------------------------------------------------
// split combine: one wave per (stream, head, block position) row
// ---------------------------------------------------------------------------

template <int D>
__device__ __forceinline__ void combine_row(const CombineArgs& c, int64_t row, int lane);

// one wave per row; the grid strides over the rows (capped grid)
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs c, int64_t rows) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4)
    combine_row<D>(c, row, lane);
}

template <int D>
__device__ __forceinline__ void combine_row(const CombineArgs& c, int64_t row, int lane) {
  // Each load instruction moves 16 bytes per lane, so one instruction covers
  // RPL partial rows (lane group q = lane / (D/4) takes split x + q, dims
  // 4*(lane % (D/4)) .. +3), and four instructions keep 4*RPL partial rows in
  // flight per wave; past the row's last split the loads are masked off.
  constexpr int LPR = D / 4;        // lanes per partial row
  constexpr int RPL = 64 / LPR;     // partial rows per load instruction
  constexpr int U = 4;              // load instructions in flight
  const int q = lane / LPR;
  const int d0 = (lane % LPR) * 4;
  const int64_t hl_out = (int64_t)c.Hq * c.Lb;
  const int b = (int)(row / hl_out);
  // partial rows of this output row: split x of its run is (x0 + x) * hl + rem
  int64_t hl = hl_out, rem = row % hl_out;
  int x0 = 0, ns = 0;
  if (c.plan) {   // masked step: only the listed pairs, each unit holding its group's G * Lb rows
    const int P = c.B * c.Hkv;
    const int h = (int)(rem / c.Lb), pos = (int)(rem % c.Lb);
    const int a = ld_const(c.plan + 5 + 2 * P, (int64_t)b * c.Hkv + h / c.G);
    if (a < 0) return;   // cache reused: the row is left untouched
    const int32_t* base = c.plan + 4 + P;
    x0 = ld_const(base, a);
    ns = ld_const(base, a + 1) - x0;
    hl = (int64_t)c.G * c.Lb;
    rem = (int64_t)(h % c.G) * c.Lb + pos;
  } else {
    for (int bb = 0; bb < b; ++bb) x0 += splits_of(c.offsets, bb, c.split_tiles, c.chunk_mode, c.n_sel, c.chunk_tiles);
    ns = splits_of(c.offsets, b, c.split_tiles, c.chunk_mode, c.n_sel, c.chunk_tiles);
  }
  if (x0 > c.total_splits) x0 = c.total_splits;
  if (ns > c.total_splits - x0) ns = c.total_splits - x0;
  const float le = c.extra_lse ? c.extra_lse[row] : kNegInf;
  // split LSEs, 64 at a time across the lanes: max first
  float mx = le;
  for (int x = lane; x < ns; x += 64) mx = fmaxf(mx, c.part_lse[(int64_t)(x0 + x) * hl + rem]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;   // this lane group's splits
  if (mx != kNegInf) {
    for (int x1 = 0; x1 < ns; x1 += 64) {
      const int nx = min(64, ns - x1);
      // lane j holds the weight of split x1 + j (0 past the last split)
      const float wl = lane < nx ? expf(c.part_lse[(int64_t)(x0 + x1 + lane) * hl + rem] - mx) : 0.f;
      for (int j = 0; j < nx; j += U * RPL) {
        float w4[U];
        f32x4 v4[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int jj = j + u * RPL + q;   // this lane's split within the 64
          w4[u] = __shfl(wl, jj < 64 ? jj : 63, 64);
          v4[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
          if (jj < nx) v4[u] = *(const f32x4*)(c.part_o + ((int64_t)(x0 + x1 + jj) * hl + rem) * D + d0);
          else w4[u] = 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          wsum += w4[u];
          acc = w4[u] * v4[u] + acc;
        }
      }
    }
  }
  // the lane groups' sums, then the extra partial
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) {
    wsum += __shfl_xor(wsum, m, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], m, 64);
  }
  if (mx != kNegInf && c.extra_lse) {
    const float w = expf(le - mx);
    wsum += w;
    acc = w * *(const f32x4*)(c.extra_o + row * D + d0) + acc;
  }
  const bool any = wsum > 0.f;
  const float inv = any ? 1.f / wsum : 0.f;
  if (q == 0) *(f32x4*)(c.o + row * D + d0) = acc * inv;
  if (lane == 0) c.lse[row] = any ? mx + logf(wsum) : kNegInf;
}

// Rows of at most kFewSplits splits, without a unit plan (the video frame's
// prefix pass: three): one row per group of D/4 lanes (4 dims each), so a
// wave combines 64 / (D/4) rows, and every load of a row -- the split LSEs,
// all partial rows and the extra partial -- is issued before the first of
// them is used: one memory round trip per row instead of two, and half (D =
// 128) or a quarter (D = 64) of the waves.  Same weights and result as
// combine_row; the splits are summed in order.
template <int D, int NSPL>
__global__ void __launch_bounds__(256) combine_few_kernel(const CombineArgs c, int64_t rows) {
  constexpr int LPR = D / 4;        // lanes per row
  constexpr int RPW = 64 / LPR;     // rows per wave
  static_assert(LPR >= NSPL, "a row's split weights live in its own lane group");
  const int lane = threadIdx.x & 63;
  const int q = lane / LPR;
  const int li = lane % LPR;
  const int d0 = 4 * li;
  const int64_t hl = (int64_t)c.Hq * c.Lb;
  for (int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW; base < rows;
       base += (int64_t)gridDim.x * 4 * RPW) {
    const int64_t row = base + q;
    const bool valid = row < rows;   // uniform over the row's lane group
    const int b = valid ? (int)(row / hl) : 0;
    const int64_t rem = row % hl;
    int x0 = 0;
    for (int bb = 0; bb < b; ++bb) x0 += splits_of(c.offsets, bb, c.split_tiles, c.chunk_mode, c.n_sel, c.chunk_tiles);
    int ns = valid ? splits_of(c.offsets, b, c.split_tiles, c.chunk_mode, c.n_sel, c.chunk_tiles) : 0;
    if (x0 > c.total_splits) x0 = c.total_splits;
    if (ns > c.total_splits - x0) ns = c.total_splits - x0;
    if (ns > NSPL) ns = NSPL;   // the host chose this kernel only when no stream has more
    // every load of the row first
    const float ls = li < ns ? c.part_lse[(int64_t)(x0 + li) * hl + rem] : kNegInf;   // lane li: split li's LSE
    f32x4 v[NSPL];
#pragma unroll
    for (int x = 0; x < NSPL; ++x) {
      v[x] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (x < ns) v[x] = *(const f32x4*)(c.part_o + ((int64_t)(x0 + x) * hl + rem) * D + d0);
    }
    const bool ext = valid && c.extra_lse != nullptr;
    const float le = ext ? c.extra_lse[row] : kNegInf;
    f32x4 ve = {0.f, 0.f, 0.f, 0.f};
    if (ext) ve = *(const f32x4*)(c.extra_o + row * D + d0);
    // max over the row's splits and the extra partial (within the lane group)
    float mx = fmaxf(ls, le);
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    const float wl = (li < ns && mx != kNegInf) ? expf(ls - mx) : 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
#pragma unroll
    for (int x = 0; x < NSPL; ++x) {
      const float w = __shfl(wl, q * LPR + x, 64);   // 0 past the row's last split
      wsum += w;
      acc = w * v[x] + acc;
    }
    if (mx != kNegInf && ext) {
      const float w = expf(le - mx);
      wsum += w;
      acc = w * ve + acc;
    }
    const bool any = wsum > 0.f;
    const float inv = any ? 1.f / wsum : 0.f;
    if (valid) {
      *(f32x4*)(c.o + row * D + d0) = acc * inv;
      if (li == 0) c.lse[row] = any ? mx + logf(wsum) : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// two-partial merge: one wave per row (all reads of a row precede its writes)
// ---------------------------------------------------------------------------

__device__ __forceinline__ void merge_row(int64_t row, int D, const float* oa, const float* la, const float* ob,
                                          const float* lb, float* o, float* lse, int lane);

// one wave per row; the grid strides over the rows (capped grid)
__global__ void __launch_bounds__(256) merge_kernel(int64_t rows, int D, const float* oa, const float* la,
                                                    const float* ob, const float* lb, float* o, float* lse) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4)
    merge_row(row, D, oa, la, ob, lb, o, lse, lane);
}

__device__ __forceinline__ void merge_row(int64_t row, int D, const float* oa, const float* la, const float* ob,
                                          const float* lb, float* o, float* lse, int lane) {
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
// adaptive reuse masks (FlashBlock explainer page, "Adaptive Reuse Strategies")
// ---------------------------------------------------------------------------
//
// Masks are [B][Hkv] int32, 1 = recompute that (stream, KV head)'s
// block-external partial at this step.  They stay on the device: the prefix
// pass and the split combine read them, so no host round trip decides a step.

// threshold-based reuse, part 1: one wave per block token -- did its K or V
// row (any KV head, any dim) change by more than eps since the previous step?
// Lanes take 16-byte vectors of the token's Hkv*D elements (8 bf16 or 4 fp32;
// base pointers and strides are 16-byte aligned), four vectors of each of the
// four tensors loaded before any is compared, so a token of 8 heads x 128 dims
// costs one memory round trip rather than one per element group.
template <typename T>
__device__ __forceinline__ void tau_flag_token(const TauArgs& t, int64_t tok, int lane);

// one wave per token; the grid strides over the tokens (capped grid)
template <typename T>
__global__ void __launch_bounds__(256) tau_flags_kernel(const TauArgs t) {
  const int lane = threadIdx.x & 63;
  const int64_t toks = (int64_t)t.B * t.Lb;
  for (int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); tok < toks; tok += (int64_t)gridDim.x * 4)
    tau_flag_token<T>(t, tok, lane);
}

template <typename T>
__device__ __forceinline__ void tau_flag_token(const TauArgs& t, int64_t tok, int lane) {
  if (t.step == 0) {   // no previous step: every token is new
    if (lane == 0) t.flags[tok] = 1;
    return;
  }
  typedef f32x4 Raw;                      // 16 bytes of T
  constexpr int VE = 16 / (int)sizeof(T);  // elements per vector
  constexpr int U = 4;                     // vectors per lane per round
  const int b = (int)(tok / t.Lb);
  const int pos = (int)(tok % t.Lb);
  const int64_t base = (int64_t)b * t.kv_sb + (int64_t)pos * t.kv_st;
  const int per_head = t.D / VE;
  const int nvec = t.Hkv * per_head;
  const T* kc = (const T*)t.k_cur + base;
  const T* kp = (const T*)t.k_prev + base;
  const T* vc = (const T*)t.v_cur + base;
  const T* vp = (const T*)t.v_prev + base;
  bool changed = false;
  for (int e0 = lane; e0 < nvec; e0 += 64 * U) {
    Raw a[U], p[U], c[U], q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * 64;
      if (e < nvec) {
        const int64_t i = (int64_t)(e / per_head) * t.kv_sh + (e % per_head) * VE;
        a[u] = *(const Raw*)(kc + i);
        p[u] = *(const Raw*)(kp + i);
        c[u] = *(const Raw*)(vc + i);
        q[u] = *(const Raw*)(vp + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (e0 + u * 64 < nvec) {
        typedef T Vec __attribute__((ext_vector_type(VE)));   // the 16 bytes as VE elements
        const Vec ka = __builtin_bit_cast(Vec, a[u]), kb = __builtin_bit_cast(Vec, p[u]);
        const Vec va = __builtin_bit_cast(Vec, c[u]), vb = __builtin_bit_cast(Vec, q[u]);
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          const float dk = fabsf((float)ka[j] - (float)kb[j]);
          const float dv = fabsf((float)va[j] - (float)vb[j]);
          changed |= dk > t.eps || dv > t.eps;
        }
      }
    }
  }
  changed = __any(changed);
  if (lane == 0) t.flags[tok] = changed ? 1 : 0;
}

// threshold-based reuse, part 2: one workgroup per stream -- M = updated
// tokens; recompute every KV head of the stream iff M >= tau (or step 0)
__global__ void __launch_bounds__(256) tau_finalize_kernel(const TauArgs t) {
  __shared__ int part[4];
  const int b = blockIdx.x;
  int m = 0;
  for (int i = threadIdx.x; i < t.Lb; i += 256) m += t.flags[(int64_t)b * t.Lb + i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m += __shfl_xor(m, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  const int total = part[0] + part[1] + part[2] + part[3];
  const int refresh = (t.step == 0 || total >= t.tau) ? 1 : 0;
  if (threadIdx.x == 0) t.count[b] = total;
  for (int g = threadIdx.x; g < t.Hkv; g += 256) t.mask[(int64_t)b * t.Hkv + g] = refresh;
}

// head-wise selection: one workgroup per (stream, KV head).  For each query
// head of the group, the cosine similarity of its block queries at the
// reference step (q_ref) and now (fp64 sums, so the threshold decision does
// not hinge on fp32 summation order); the KV head is recomputed iff some
// similarity is <= gamma (or step 0), and then the group's q_ref rows take
// the current queries.  Rows move as 8-element (16- or 32-byte) vectors.
template <typename T>
__device__ __forceinline__ void ld8(const T* p, double* out) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (double)(float)v[j];
  } else {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[j] = a[j];
      out[4 + j] = b[j];
    }
  }
}

template <typename T>
__device__ void gamma_group(const GammaArgs& a) {
  constexpr int NT = 1024;
  __shared__ double red[3][NT / 64];
  const int b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int cs = a.D == 128 ? 4 : 3;   // log2 of 8-element chunks per row
  const int nv = a.Lb << cs;           // 8-element chunks per head
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const T* qc = (const T*)a.q_cur;
  T* qr = (T*)a.q_ref;
  bool refresh = a.step == 0;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    double dot = 0.0, n1 = 0.0, n2 = 0.0;
    for (int i = threadIdx.x; i < nv; i += NT) {
      const int pos = i >> cs, c8 = (i & ((1 << cs) - 1)) * 8;
      double x[8], y[8];
      ld8(qr + (((int64_t)b * a.Lb + pos) * a.Hq + h) * a.D + c8, x);
      ld8(qc + (int64_t)b * a.q_sb + (int64_t)pos * a.q_st + (int64_t)h * a.q_sh + c8, y);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        dot = fma(x[j], y[j], dot);
        n1 = fma(x[j], x[j], n1);
        n2 = fma(y[j], y[j], n2);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      dot += __shfl_xor(dot, o, 64);
      n1 += __shfl_xor(n1, o, 64);
      n2 += __shfl_xor(n2, o, 64);
    }
    if (lane == 0) {
      red[0][wave] = dot;
      red[1][wave] = n1;
      red[2][wave] = n2;
    }
    __syncthreads();
    double sd = 0.0, s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      sd += red[0][w];
      s1 += red[1][w];
      s2 += red[2][w];
    }
    const double sim = (s1 > 0.0 && s2 > 0.0) ? sd / sqrt(s1 * s2) : 0.0;
    if (threadIdx.x == 0) a.sim[(int64_t)b * a.Hq + h] = (float)sim;
    refresh |= !(sim > (double)a.gamma);
    __syncthreads();   // red is reused by the next head
  }
  if (threadIdx.x == 0) a.mask[(int64_t)b * a.Hkv + g] = refresh ? 1 : 0;
  if (!refresh) return;
  for (int i = threadIdx.x; i < G * nv; i += NT) {   // 16-byte moves
    const int h = g * G + i / nv, r = i % nv;
    const int pos = r >> cs, c8 = (r & ((1 << cs) - 1)) * 8;
    const T* src = qc + (int64_t)b * a.q_sb + (int64_t)pos * a.q_st + (int64_t)h * a.q_sh + c8;
    T* dst = qr + (((int64_t)b * a.Lb + pos) * a.Hq + h) * a.D + c8;
    if constexpr (sizeof(T) == 2) {
      *(bf16x8*)dst = *(const bf16x8*)src;
    } else {
      *(f32x4*)dst = *(const f32x4*)src;
      *(f32x4*)(dst + 4) = *(const f32x4*)(src + 4);
    }
  }
}

__global__ void __launch_bounds__(1024) gamma_kernel(const GammaArgs a) {
  if (a.dtype == kDtypeBf16)
    gamma_group<__bf16>(a);
  else
    gamma_group<float>(a);
}

// ---------------------------------------------------------------------------
// finalised block -> prefix KV cache: one thread per 16-byte piece of a row
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) append_kernel(const AppendArgs a) {
  const int pieces = a.D * a.esize / 16;   // 16-byte pieces per (token, KV head) row
  const int64_t per_tensor = (int64_t)a.B * a.Lb * a.Hkv * pieces;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < 2 * per_tensor; j += (int64_t)gridDim.x * 256) {
  int64_t i = j;
  const bool is_v = i >= per_tensor;
  if (is_v) i -= per_tensor;
  const int pc = (int)(i % pieces);
  int64_t r = i / pieces;
  const int g = (int)(r % a.Hkv);
  r /= a.Hkv;
  const int t = (int)(r % a.Lb);
  const int b = (int)(r / a.Lb);
  const int64_t src = (int64_t)b * a.kv_sb + (int64_t)t * a.kv_st + (int64_t)g * a.kv_sh;
  const int64_t dst = (ld_const(a.dst_rows, b) + t) * a.pre_st + (int64_t)g * a.pre_sh;
  const char* s = (const char*)(is_v ? a.v_blk : a.k_blk) + src * a.esize + pc * 16;
  char* d = (char*)(is_v ? a.v_pre : a.k_pre) + dst * a.esize + pc * 16;
  *(f32x4*)d = *(const f32x4*)s;
  }
}

// ---------------------------------------------------------------------------
// chunk selection for the sparse variant (pooled key, max query score, top-k)
// ---------------------------------------------------------------------------
//
// Pooled keys live in [B][chunk_cap][Hkv][D] fp32, scores in [B][Hkv][chunk_cap]
// fp32, so that a caller can keep the pooled keys of an append-only prefix
// and pool only the chunks a new block touched.

__device__ __forceinline__ int chunks_of(const int64_t* off, int b, int cl) {
  return (int)((prefix_len(off, b) + cl - 1) / cl);
}

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// one wave per (stream, chunk, KV head): the mean of the chunk's keys in fp32.
// A lane loads 16 bytes of a key row, so one load instruction covers 64 / P
// rows (P = 16-byte pieces per row); four such loads are in flight at once.
template <int D, typename T>
__device__ __forceinline__ void pool_chunk(const SelectArgs& a, int b, int c, int g, int lane) {
  constexpr int EPP = 16 / (int)sizeof(T);
  constexpr int P = D / EPP;
  constexpr int RPL = 64 / P;
  typedef T vecT __attribute__((ext_vector_type(EPP)));
  const int64_t s1 = ld_const(a.offsets, b + 1);
  const int64_t t0 = ld_const(a.offsets, b) + (int64_t)c * a.chunk_len;
  const int64_t t1 = min(t0 + a.chunk_len, s1);
  const int row = lane / P, piece = lane % P;
  const T* base = (const T*)a.k_pre + (int64_t)g * a.pre_sh + piece * EPP;
  float acc[EPP];
#pragma unroll
  for (int j = 0; j < EPP; ++j) acc[j] = 0.f;
  int64_t t = t0 + row;
  for (; t + 3 * RPL < t1; t += 4 * RPL) {
    vecT v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *(const vecT*)(base + (t + u * RPL) * a.pre_st);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < EPP; ++j) acc[j] += to_f32(v[u][j]);
  }
  for (; t < t1; t += RPL) {
    const vecT v = *(const vecT*)(base + t * a.pre_st);
#pragma unroll
    for (int j = 0; j < EPP; ++j) acc[j] += to_f32(v[j]);
  }
#pragma unroll
  for (int o = P; o < 64; o <<= 1)
#pragma unroll
    for (int j = 0; j < EPP; ++j) acc[j] += shfl_xor_f(acc[j], o);
  if (lane < P) {
    const float inv = 1.f / (float)(t1 - t0);
    float* dst = a.pooled + (((int64_t)b * a.chunk_cap + c) * a.Hkv + g) * D + piece * EPP;
#pragma unroll
    for (int j = 0; j < EPP; j += 4) *(f32x4*)(dst + j) = (f32x4){acc[j] * inv, acc[j + 1] * inv,
                                                                  acc[j + 2] * inv, acc[j + 3] * inv};
  }
}

// grid: 4 waves per workgroup over (stream, chunk first_chunk.., KV head)
__global__ void __launch_bounds__(256) pool_kernel(const SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int span = a.max_chunks - a.first_chunk;
  const int64_t n = (int64_t)a.B * span * a.Hkv;
  for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < n; w += (int64_t)gridDim.x * 4) {
    const int g = (int)(w % a.Hkv);
    const int64_t r = w / a.Hkv;
    const int c = a.first_chunk + (int)(r % span), b = (int)(r / span);
    if (c >= chunks_of(a.offsets, b, a.chunk_len)) continue;   // wave-uniform
    if (a.dtype == kDtypeBf16) {
      if (a.D == 128) pool_chunk<128, __bf16>(a, b, c, g, lane); else pool_chunk<64, __bf16>(a, b, c, g, lane);
    } else {
      if (a.D == 128) pool_chunk<128, float>(a, b, c, g, lane); else pool_chunk<64, float>(a, b, c, g, lane);
    }
  }
}

// x == hi + mid + lo exactly: each bf16 term takes the next 8 significand bits
__device__ __forceinline__ void split3(const float* x, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    const float r1 = x[j] - (float)h;
    const __bf16 m = (__bf16)r1;
    hi[j] = h;
    mid[j] = m;
    lo[j] = (__bf16)(r1 - (float)m);
  }
}

// bf16 queries: S[q row][chunk] = Q . pooled on MFMA, the fp32 pooled key
// split into three bf16 terms.  bf16 x bf16 products are exact in fp32, so
// the score carries fp32 accumulation error only.  A workgroup scores 64
// chunks, 16 per wave (B operand columns, held in registers), against all
// G*Lb query rows of its KV head (A operand), which pass through LDS in
// 64-row rounds shared by the four waves: the next round's rows are loaded
// into registers while the current round's MFMAs run.  LDS row of 2D bytes,
// 16-byte slot j of row r stored at slot j ^ (r mod slots-per-row), so the 16
// rows read by one fragment load fall on distinct banks.
template <int D>
__device__ __forceinline__ void score_mfma(const SelectArgs& a, int b, int g, int c_wg, int n) {
  constexpr int KS = D / 32, SLOTS = D / 8, ROWB = 2 * D;
  constexpr int PER = 64 * SLOTS / 256;   // 16-byte slots staged per thread per round
  __shared__ __attribute__((aligned(16))) char qs[2][64 * ROWB];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, lg = lane >> 4, wave = tid >> 6;
  const int c = c_wg + wave * 16 + l16;
  bf16x8 kh[KS], km[KS], kl[KS];
  if (c < n) {
    const float* pk = a.pooled + (((int64_t)b * a.chunk_cap + c) * a.Hkv + g) * D + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4 x0 = *(const f32x4*)(pk + ks * 32), x1 = *(const f32x4*)(pk + ks * 32 + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      split3(x, kh[ks], km[ks], kl[ks]);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kh[ks] = km[ks] = kl[ks] = (bf16x8){};
  }
  const int rows = a.G * a.Lb;
  const int rounds = (rows + 63) / 64;
  u32x4 stage[PER];
  auto load = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + 256 * j, row = r * 64 + i / SLOTS, slot = i % SLOTS;
      if (row < rows) {
        const int h = g * a.G + row / a.Lb, pos = row % a.Lb;
        stage[j] = *(const u32x4*)((const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)pos * a.q_st +
                                   (int64_t)h * a.q_sh + slot * 8);
      } else {
        stage[j] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + 256 * j, rr = i / SLOTS, slot = i % SLOTS;
      *(u32x4*)(qs[buf] + rr * ROWB + ((slot ^ (rr & (SLOTS - 1))) * 16)) = stage[j];
    }
  };
  load(0);
  store(0);
  __syncthreads();
  float best = kNegInf;
  for (int r = 0; r < rounds; ++r) {
    if (r + 1 < rounds) load(r + 1);
    bf16x8 qa[4][KS];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int rr = rt * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qa[rt][ks] = *(const bf16x8*)(qs[r & 1] + rr * ROWB + (((ks * 4 + lg) ^ (rr & (SLOTS - 1))) * 16));
    }
    f32x4 acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt][ks], kl[ks], acc[rt], 0, 0, 0);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt][ks], km[ks], acc[rt], 0, 0, 0);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt][ks], kh[ks], acc[rt], 0, 0, 0);
    }
    // accumulator element i of lane (l16, lg): query row 4*lg + i of the tile, chunk l16
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (r * 64 + rt * 16 + 4 * lg + i < rows) best = fmaxf(best, acc[rt][i]);
    if (r + 1 < rounds) store((r + 1) & 1);
    __syncthreads();
  }
  best = fmaxf(best, shfl_xor_f(best, 16));
  best = fmaxf(best, shfl_xor_f(best, 32));
  if (lg == 0 && c < n) a.scores[((int64_t)b * a.Hkv + g) * a.chunk_cap + c] = best;
}

// fp32 queries: plain fp32 dot products, four lanes per chunk splitting the
// query rows, then the max over them
template <int D>
__device__ __forceinline__ void score_f32(const SelectArgs& a, int b, int g, int tile0, int n) {
  const int c = tile0 + (threadIdx.x >> 2), sub = threadIdx.x & 3;
  const bool live = c < n;
  const float* pk = a.pooled + (((int64_t)b * a.chunk_cap + (live ? c : 0)) * a.Hkv + g) * D;
  float kk[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const f32x4 v = *(const f32x4*)(pk + d);
    kk[d] = v[0]; kk[d + 1] = v[1]; kk[d + 2] = v[2]; kk[d + 3] = v[3];
  }
  float best = kNegInf;
  const int rows = a.G * a.Lb;
  for (int r = sub; r < rows; r += 4) {
    const int h = g * a.G + r / a.Lb, pos = r % a.Lb;
    const float* qp = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)pos * a.q_st + (int64_t)h * a.q_sh;
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const f32x4 qv = *(const f32x4*)(qp + d);
#pragma unroll
      for (int j = 0; j < 4; ++j) dot = __builtin_fmaf(qv[j], kk[d + j], dot);
    }
    best = fmaxf(best, dot);
  }
  best = fmaxf(best, shfl_xor_f(best, 1));
  best = fmaxf(best, shfl_xor_f(best, 2));
  if (live && sub == 0) a.scores[((int64_t)b * a.Hkv + g) * a.chunk_cap + c] = best;
}

// one workgroup per (stream, KV head, 64 chunks)
template <bool BF16>
__global__ void __launch_bounds__(256) score_kernel(const SelectArgs a) {
  constexpr int CPW = 64;
  const int tiles = (a.max_chunks + CPW - 1) / CPW;
  const int tile = blockIdx.x % tiles;
  const int g = (blockIdx.x / tiles) % a.Hkv, b = blockIdx.x / tiles / a.Hkv;
  const int n = chunks_of(a.offsets, b, a.chunk_len);
  if (tile * CPW >= n) return;   // uniform over the workgroup
  if constexpr (BF16) {
    if (a.D == 128) score_mfma<128>(a, b, g, tile * CPW, n); else score_mfma<64>(a, b, g, tile * CPW, n);
  } else {
    if (a.D == 128) score_f32<128>(a, b, g, tile * CPW, n); else score_f32<64>(a, b, g, tile * CPW, n);
  }
}

// order key: ascending order = descending score (-0 counted as +0)
__device__ __forceinline__ uint32_t rank_key(float s) {
  if (s == 0.f) s = 0.f;
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  return ~((u & 0x80000000u) ? ~u : (u | 0x80000000u));
}

// exclusive prefix sum of v over the threads of the workgroup (at most 1024)
__device__ __forceinline__ int wg_exclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();   // wsum free from any earlier use
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
  return before + incl - v;
}

// one workgroup per (stream, KV head): radix select of the k-th best order
// key (four 8-bit digits, most significant first), then the chunks strictly
// better plus the lowest-index chunks tied with it, written ascending
__global__ void __launch_bounds__(1024) topk_kernel(const SelectArgs a) {
  __shared__ uint32_t keys[kMaxSelectChunks];
  __shared__ int hist[256];
  __shared__ int wsum[16];
  __shared__ uint32_t sel_prefix;
  __shared__ int sel_rank;
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = chunks_of(a.offsets, b, a.chunk_len);
  const float* sc = a.scores + ((int64_t)b * a.Hkv + g) * a.chunk_cap;
  for (int i = tid; i < n; i += 1024) keys[i] = rank_key(sc[i]);
  if (tid == 0) {
    sel_prefix = 0;
    sel_rank = a.k;   // 1-based rank of the wanted key among those matching the prefix
  }
  uint32_t mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = sel_prefix;
    for (int i = tid; i < n; i += 1024) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {   // wave 0: the digit whose cumulative count reaches the rank
      const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const int sum4 = h0 + h1 + h2 + h3;
      int incl = sum4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int rank = sel_rank;
      const int excl = incl - sum4;
      if (excl < rank && rank <= incl) {   // exactly one lane
        int cum = excl, d = 4 * lane;
        const int hs[4] = {h0, h1, h2, h3};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (d == 4 * lane + j && rank > cum + hs[j]) {
            cum += hs[j];
            d = 4 * lane + j + 1;
          }
        }
        sel_prefix = prefix | ((uint32_t)d << shift);
        sel_rank = rank - cum;
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t thr = sel_prefix;   // the k-th best key
  const int ties_wanted = sel_rank;  // how many keys equal to it are kept (lowest indices)
  // compaction in index order over contiguous runs of chunks per thread
  const int per = (n + 1023) / 1024;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  int ties = 0;
  for (int i = i0; i < i1; ++i) ties += keys[i] == thr;
  int tie_rank = wg_exclusive_scan(ties, wsum);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    if (key < thr) ++cnt;
    else if (key == thr) cnt += tie_rank++ < ties_wanted;
  }
  int pos = wg_exclusive_scan(cnt, wsum);
  tie_rank -= ties;
  int32_t* out = a.idx_out + ((int64_t)b * a.Hkv + g) * a.k;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    bool take = key < thr;
    if (key == thr) take = tie_rank++ < ties_wanted;
    if (take) out[pos++] = i;
  }
}

// ---------------------------------------------------------------------------
// debug check of a cached partial before a reuse step: *flag = 1 if any value
// is NaN (every writer stores the same 1, so the race is benign)
// ---------------------------------------------------------------------------

__global__ void flag_clear_kernel(int32_t* flag) {
  if (threadIdx.x == 0) *flag = 0;
}

__global__ void __launch_bounds__(256) nan_scan_kernel(const float* x, int64_t n, int32_t* flag) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    bad |= __builtin_isnan(x[i]);
  if (bad) *flag = 1;
}

// debug check of a sparse chunk list [B][Hkv][k]: *flag = 1 unless every
// (stream, KV head) list is strictly ascending with 0 <= c < the stream's
// chunk count (the flag is cleared first)
__global__ void __launch_bounds__(256) chunk_check_kernel(const int32_t* list, const int64_t* offsets, int32_t B,
                                                          int32_t Hkv, int32_t k, int32_t chunk_len, int32_t* flag) {
  bool bad = false;
  const int64_t n = (int64_t)B * Hkv * k;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int b = (int)(i / ((int64_t)Hkv * k));
    const int j = (int)(i % k);
    const int32_t c = list[i];
    bad |= c < 0 || c >= chunks_of(offsets, b, chunk_len) || (j > 0 && list[i - 1] >= c);
  }
  if (bad) *flag = 1;
}

// ---------------------------------------------------------------------------
// unit plan of a masked step: one 256-thread workgroup
// ---------------------------------------------------------------------------
//
// Lists the (stream, KV head) pairs the mask recomputes, in mask order, and
// sizes their splits so that just those pairs fill the workgroups the
// all-heads plan would use (cap): the smallest split length (>= min_split
// tiles) whose workgroups fit, or one split per pair.  A step that recomputes
// 2 of 12 heads then runs in about 2/12 of a full pass instead of leaving 10/12
// of the workgroups idle.  Layout: see plan_ints in fb_internal.h.
//
// Thread t takes pairs t, t + 256, ...; the first of them stays in registers
// between the phases (all of them when B * Hkv <= 256), the others are read
// again.  The mask and the stream's tile count are loaded together, so a step
// with few pairs costs two dependent memory round trips and a handful of
// barriers.

constexpr int kPlanThreads = 256;

// sum and max over the workgroup in one exchange; red holds 2 * waves values
__device__ __forceinline__ void wg_sum_max64(int64_t& s, int64_t& m, int64_t* red) {
  constexpr int kWaves = kPlanThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    s += __shfl_xor(s, o, 64);
    const int64_t other = __shfl_xor(m, o, 64);
    m = other > m ? other : m;
  }
  __syncthreads();   // red free from any earlier use
  if (lane == 0) {
    red[wave] = s;
    red[kWaves + wave] = m;
  }
  __syncthreads();
  s = 0;
  m = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    s += red[w];
    m = red[kWaves + w] > m ? red[kWaves + w] : m;
  }
}

__device__ __forceinline__ int wg_total(const int* wsum) {
  int t = 0;
#pragma unroll
  for (int w = 0; w < kPlanThreads / 64; ++w) t += wsum[w];
  return t;
}

__global__ void __launch_bounds__(kPlanThreads) unit_plan_kernel(const UnitPlanArgs u) {
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ int64_t red[2 * (kPlanThreads / 64)];
  const int P = u.B * u.Hkv;
  int32_t* act = u.plan + 4;
  int32_t* base = act + P;
  int32_t* slot = base + P + 1;
  const int tid = threadIdx.x;
  // this thread's pair in a chunk: recomputed?, and its stream's tile count
  // (0 if not recomputed); the first chunk's values stay in registers
  int on0 = 0, slot0 = -1;
  int64_t t0 = 0;
  auto pair = [&](int c0, int& on, int64_t& t) {
    if (c0 == 0) {
      on = on0;
      t = t0;
      return;
    }
    const int i = c0 + tid;
    on = i < P && u.mask[i] != 0;
    t = on ? (prefix_len(u.offsets, i / u.Hkv) + kTile - 1) / kTile : 0;
  };
  if (tid < P) {   // both loads in flight together
    const int64_t lp = prefix_len(u.offsets, tid / u.Hkv);
    on0 = u.mask[tid] != 0;
    t0 = on0 ? (lp + kTile - 1) / kTile : 0;
  }
  // the listed pairs, in mask order; total and longest tile count
  int n = 0;
  int64_t tot = 0, mx = 0;
  for (int c0 = 0; c0 < P; c0 += kPlanThreads) {
    int on;
    int64_t t;
    pair(c0, on, t);
    const int pos = wg_exclusive_scan(on, wsum);
    const int i = c0 + tid;
    const int sl = on ? n + pos : -1;
    if (i < P) slot[i] = sl;
    if (c0 == 0) slot0 = sl;
    if (on) act[n + pos] = i;
    n += wg_total(wsum);
    tot += t;
    mx = t > mx ? t : mx;
  }
  if (n == 0) {   // nothing recomputed (uniform): an empty plan, no split search
    if (tid == 0) {
      base[0] = 0;
      u.plan[0] = 0;
      u.plan[1] = u.min_split;
      u.plan[2] = 0;
      u.plan[3] = 0;
    }
    return;
  }
  wg_sum_max64(tot, mx, red);
  // split length: total tiles of the listed pairs over the cap, raised until
  // their splits' workgroups fit (or one split per pair)
  int64_t st = ((tot * u.row_tiles) + u.cap - 1) / (u.cap > 0 ? u.cap : 1);
  if (st < u.min_split) st = u.min_split;
  for (;;) {
    int64_t units = 0, unused = 0;
    for (int c0 = 0; c0 < P; c0 += kPlanThreads) {
      int on;
      int64_t t;
      pair(c0, on, t);
      units += (t + st - 1) / st;   // 0 for a pair that is not recomputed
    }
    wg_sum_max64(units, unused, red);
    if (units * u.row_tiles <= u.cap || st >= mx) break;   // uniform over the workgroup
    ++st;
  }
  // first unit of each listed pair (the scan runs in mask order, which is the
  // listed order)
  int done = 0;
  for (int c0 = 0; c0 < P; c0 += kPlanThreads) {
    int on;
    int64_t t;
    pair(c0, on, t);
    const int ns = on ? (int)((t + st - 1) / st) : 0;
    const int pos = wg_exclusive_scan(ns, wsum);
    if (on) base[c0 == 0 ? slot0 : slot[c0 + tid]] = done + pos;
    done += wg_total(wsum);
  }
  if (tid == 0) {
    base[n] = done;
    u.plan[0] = done * u.row_tiles;
    u.plan[1] = (int)st;
    u.plan[2] = n;
    u.plan[3] = done;
  }
}

// ---------------------------------------------------------------------------
// scratch of the no-allocation step (fb_step_noalloc)
// ---------------------------------------------------------------------------
//
// The split partials of the prefix pass normally live in a caller workspace.
// For callers that cannot allocate, they live here instead: every GPU the
// library runs on holds this array from the module's load until the process
// ends, and every call on that GPU shares it.  In host code the array's name
// is only a host-side stand-in: its device address on each GPU comes from
// hipGetSymbolAddress with that GPU current, and only that address is passed
// to kernels.

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

int noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// 1-D grids of the row/element kernels are capped, and those kernels stride
// over what the grid does not cover: a dispatch's work-item count stays far
// inside its 32-bit limit for any size the host accepts.
constexpr int64_t kMaxBlocks = 1 << 20;
static dim3 capped_grid(int64_t blocks) { return dim3((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks)); }

template <int D, int QT, int NW, int NS, int WPC, bool P, int RW, int KG>
static int launch_bf16(const AttnArgs& a, hipStream_t s) {
  constexpr int minw = (NW * WPC + 3) / 4;   // waves per SIMD when WPC workgroups share a CU
  hipLaunchKernelGGL((attn_bf16<D, QT, NW, NS, minw, P, RW, KG>), dim3(a.grid), dim3(64 * NW), 0, s, a);
  return (int)hipGetLastError();
}

template <int D, bool P>
static int launch_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_f32m<D, P>), dim3(a.grid), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

template <int D>
static int launch_bf16_cfg(const AttnArgs& a, int cfg, hipStream_t s) {
  switch (cfg) {
#define FB_CFG_LAUNCH(ID, QT, NW, NS, WPC, PART, RW, KG) \
    case ID: return launch_bf16<D, QT, NW, NS, WPC, (PART) != 0, RW, KG>(a, s);
    FB_BF16_CFGS(FB_CFG_LAUNCH)
#undef FB_CFG_LAUNCH
    default: return (int)hipErrorInvalidValue;
  }
}

int launch_attn(const AttnArgs& a, int dtype, int head_dim, int cfg, bool partial, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.grid == 0) return 0;
  if (dtype == 0) {  // fp32
    if (head_dim == 64) return partial ? launch_f32<64, true>(a, s) : launch_f32<64, false>(a, s);
    return partial ? launch_f32<128, true>(a, s) : launch_f32<128, false>(a, s);
  }
  return head_dim == 64 ? launch_bf16_cfg<64>(a, cfg, s) : launch_bf16_cfg<128>(a, cfg, s);
}

#ifndef FB_COMBINE_MANY
#define FB_COMBINE_MANY 1
#endif
constexpr int64_t kFewRowsManySplits = 4096;   // rows up to which 17-32 splits go in one round trip
int launch_combine(const CombineArgs& c, int64_t rows, void* stream) {
  if (rows == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  // every load of a row in one round trip (combine_few_kernel): rows of at
  // most 4 splits, and at head_dim 128 few rows (at most 4096) of 17-32
  // splits, where one wave per row leaves the CUs nearly empty.  Measured on
  // MI355X (graph-replayed): video frame, 3 splits, 12.0 -> 7.5 us; 128K
  // GQA, 32 splits x 2048 rows, 7.95 -> 6.37; the sparse step's 30 selected
  // splits 6.5 -> 5.3; slower at 16 splits x 1024 rows (32K MHA, 4.2 -> 4.5)
  // and 8 splits x 8192 rows (the ragged batch, 9.55 -> 9.67), which keep
  // one wave per row.
  const bool many = c.D == 128 && rows <= kFewRowsManySplits && c.max_splits > 16 && c.max_splits <= 32;
  if (!c.plan && (c.max_splits <= kFewSplits || (FB_COMBINE_MANY && many))) {
    const int64_t rpw = c.D == 64 ? 4 : 2;   // rows per wave
    const dim3 grid = capped_grid((rows + 4 * rpw - 1) / (4 * rpw));
    if (c.max_splits <= kFewSplits) {
      if (c.D == 64)
        hipLaunchKernelGGL((combine_few_kernel<64, kFewSplits>), grid, dim3(256), 0, s, c, rows);
      else
        hipLaunchKernelGGL((combine_few_kernel<128, kFewSplits>), grid, dim3(256), 0, s, c, rows);
    } else {
      hipLaunchKernelGGL((combine_few_kernel<128, 32>), grid, dim3(256), 0, s, c, rows);
    }
    return (int)hipGetLastError();
  }
  const dim3 grid = capped_grid((rows + 3) / 4);
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
  hipLaunchKernelGGL(merge_kernel, capped_grid((rows + 3) / 4), dim3(256), 0, s, rows, head_dim, oa, la,
                     ob, lb, o, lse);
  return (int)hipGetLastError();
}

int launch_tau(const TauArgs& t, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t toks = (int64_t)t.B * t.Lb;
  if (t.dtype == kDtypeBf16)
    hipLaunchKernelGGL(tau_flags_kernel<__bf16>, capped_grid((toks + 3) / 4), dim3(256), 0, s, t);
  else
    hipLaunchKernelGGL(tau_flags_kernel<float>, capped_grid((toks + 3) / 4), dim3(256), 0, s, t);
  hipLaunchKernelGGL(tau_finalize_kernel, dim3((unsigned)t.B), dim3(256), 0, s, t);
  return (int)hipGetLastError();
}

int launch_append(const AppendArgs& a, void* stream) {
  const int64_t n = 2LL * a.B * a.Lb * a.Hkv * (a.D * a.esize / 16);
  hipLaunchKernelGGL(append_kernel, capped_grid((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_pool(const SelectArgs& a, void* stream) {
  const int64_t waves = (int64_t)a.B * (a.max_chunks - a.first_chunk) * a.Hkv;
  if (waves <= 0) return 0;
  hipLaunchKernelGGL(pool_kernel, capped_grid((waves + 3) / 4), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_select_pooled(const SelectArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.dtype == kDtypeBf16) {
    const int64_t tiles = (int64_t)a.B * a.Hkv * ((a.max_chunks + 63) / 64);
    hipLaunchKernelGGL(score_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, s, a);
  } else {
    const int64_t tiles = (int64_t)a.B * a.Hkv * ((a.max_chunks + 63) / 64);
    hipLaunchKernelGGL(score_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((int64_t)a.B * a.Hkv)), dim3(1024), 0, s, a);
  return (int)hipGetLastError();
}

int launch_nan_scan(const float* x, int64_t n, int32_t* flag, bool clear, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (clear) hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(64), 0, s, flag);
  if (n > 0) {
    const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(nan_scan_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n, flag);
  }
  return (int)hipGetLastError();
}

int launch_chunk_check(const int32_t* list, const int64_t* offsets, int32_t B, int32_t Hkv, int32_t k,
                       int32_t chunk_len, int32_t* flag, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(64), 0, s, flag);
  const int64_t n = (int64_t)B * Hkv * k;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(chunk_check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, list, offsets, B, Hkv, k,
                     chunk_len, flag);
  return (int)hipGetLastError();
}

int launch_unit_plan(const UnitPlanArgs& u, void* stream) {
  hipLaunchKernelGGL(unit_plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream, u);
  return (int)hipGetLastError();
}

int launch_gamma(const GammaArgs& g, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(gamma_kernel, dim3((unsigned)((int64_t)g.B * g.Hkv)), dim3(1024), 0, s, g);
  return (int)hipGetLastError();
}

}  // namespace fb
