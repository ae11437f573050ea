/*
 * flashblock.h -- C ABI of libflashblock.so: the FlashBlock attention step for
 * block diffusion on MI355X (gfx950).
 *
 * What is computed.  In block diffusion the queries of the active block attend
 * to the KV cache of all earlier, finalised blocks (the prefix, J_out) and to
 * the block's own keys and values (J_in).  FlashBlock (explainer page
 * "FlashBlock: Attention Caching for Efficient Long-Context Block Diffusion",
 * Technical Summary section 2, "Core Mechanism") splits the attention output
 * into a block-external partial A_out with log-normaliser L_out = log Z_out and
 * a block-internal partial A_in with L_in, keeps (A_out, L_out) from an earlier
 * denoising step, recomputes only A_in, and recombines them exactly with the
 * page's merge equation
 *     m = max(L_out, L_in),
 *     A = (e^(L_out-m) A_out + e^(L_in-m) A_in) / (e^(L_out-m) + e^(L_in-m)).
 * The sparse variant (same page, "Adaptive Reuse Strategies", compatibility
 * with sparse attention) caches the contribution of the keys a sparse selector
 * leaves out as a residual partial and merges it with a fresh partial over the
 * selected keys.
 *
 * Conventions (readings of points the pages leave open):
 *   - softmax scale 1/sqrt(D) unless fb_desc.softmax_scale > 0;
 *   - every L / LSE crossing this ABI is a natural log; an empty key set has
 *     A = 0 and L = -inf;
 *   - attention inside the block is bidirectional (no mask);
 *   - query head h reads KV head h / (hq / hkv).
 *
 * Layouts (element strides; the head_dim axis is always contiguous):
 *   q_blk  [B][Lb][Hq][D]   strides q_stride_{b,t,h}        dtype
 *   k_blk, v_blk [B][Lb][Hkv][D]  strides kv_stride_{b,t,h}  dtype
 *   k_pre, v_pre  packed ragged prefix: row t of KV head g of stream b sits at
 *                 base + (off[b] + t) * pre_stride_t + g * pre_stride_h
 *                 (token-major [T][Hkv][D] and head-major [Hkv][T][D] both fit)
 *   o      [B][Lb][Hq][D]   contiguous                      dtype
 *   o_ext / o_res caches [B][Hq][Lb][D] contiguous fp32;
 *   lse_ext / lse_res / lse_out [B][Hq][Lb] contiguous fp32.
 *
 * Ownership.  The caller allocates and owns every buffer (inputs, outputs,
 * caches, workspace, device offsets).  The library never allocates or frees
 * device memory and keeps no state between calls.  All device work is
 * enqueued asynchronously on the caller's stream (`stream` is a hipStream_t
 * passed as void*; NULL is the null stream); nothing synchronises except the
 * opt-in FB_DEBUG check of fb_step.
 *
 * Errors.  Arguments are validated before anything is enqueued: on an error
 * nothing is launched, outputs are untouched, the status code says which check
 * failed and fb_last_error() (thread-local) gives the detail.  Size limits:
 * batch * hkv <= 2^21, batch * hq * block_len <= 2^30, and each attention pass
 * at most 2^22 workgroups (FB_ERR_SHAPE beyond them), so that every launch's
 * grid stays inside the dispatch limits.  A launch failure
 * returns FB_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronisation.  No C++ exception crosses this interface.
 */
#ifndef FLASHBLOCK_H
#define FLASHBLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FB_ABI_VERSION 1

typedef int32_t fb_status;
enum {
  FB_OK = 0,
  FB_ERR_NULL = 1,        /* a required pointer is NULL */
  FB_ERR_SHAPE = 2,       /* inconsistent sizes: hq % hkv, batch, block_len, offsets, strides */
  FB_ERR_ALIGN = 3,       /* a base pointer or stride breaks 16-byte row alignment */
  FB_ERR_WORKSPACE = 4,   /* workspace smaller than fb_workspace_size() */
  FB_ERR_UNSUPPORTED = 5, /* dtype or head_dim not built */
  FB_ERR_ARG = 6,         /* bad step, refresh period, mode or chunk list */
  FB_ERR_HIP = 7          /* the HIP runtime refused a launch */
};

enum { FB_F32 = 0, FB_BF16 = 1 };
enum { FB_MODE_CACHED = 0, FB_MODE_FULL = 1 };
enum { FB_CHUNKS_SELECTED = 1, FB_CHUNKS_COMPLEMENT = 2 };

/* Shapes, strides and prefix offsets shared by every call. */
typedef struct fb_desc {
  int32_t abi_version;      /* must equal FB_ABI_VERSION */
  int32_t dtype;            /* FB_F32 or FB_BF16: q/k/v (block and prefix) and o */
  int32_t batch;            /* B >= 1 independent streams */
  int32_t hq;               /* query heads */
  int32_t hkv;              /* KV heads; hq % hkv == 0 */
  int32_t head_dim;         /* D: 64 or 128 */
  int32_t block_len;        /* Lb >= 1 tokens in the active block */
  float softmax_scale;      /* <= 0 selects 1/sqrt(D) */
  const int64_t* prefix_offsets_host; /* [B+1] host copy: stream b owns prefix rows
                                         off[b] .. off[b+1]-1; off[0] >= 0, non-decreasing */
  const int64_t* prefix_offsets_dev;  /* [B+1] device copy of the same values */
  int64_t q_stride_b, q_stride_t, q_stride_h;    /* q_blk */
  int64_t kv_stride_b, kv_stride_t, kv_stride_h; /* k_blk, v_blk */
  int64_t pre_stride_t, pre_stride_h;            /* k_pre, v_pre */
} fb_desc;

/* Chunk list of the sparse variant: the prefix is cut into chunks of chunk_len
 * tokens (the last one of a stream may be shorter); for each (stream, KV head)
 * `k` chunk indices are listed, ascending and unique, each < ceil(Lp_b/chunk_len).
 * SELECTED attends to the listed chunks only, COMPLEMENT to every other prefix
 * token (the unselected keys whose contribution is cached as the residual).
 * The kernels do not check the lists (an index outside the stream selects
 * nothing); with FB_DEBUG=1 in the environment, fb_step, fb_step_noalloc,
 * fb_prefix_attn and fb_prefix_partials check them on the device first (the
 * flag in the first word of the workspace, waiting on the stream; skipped
 * while the stream is being captured) and return FB_ERR_ARG before launching
 * anything else if a list breaks this contract. */
typedef struct fb_sparse {
  const int32_t* chunk_idx_dev; /* [B][Hkv][k] int32, device */
  int32_t k;                    /* chunks listed per (stream, KV head), >= 1 */
  int32_t chunk_len;            /* a positive multiple of 64 */
  int32_t mode;                 /* FB_CHUNKS_SELECTED or FB_CHUNKS_COMPLEMENT */
} fb_sparse;

/* Bytes of workspace fb_prefix_attn / fb_step / fb_step_masked /
 * fb_refresh_mask_tau need for this shape (split-KV partials, tau flags).
 * `sp` may be NULL (dense prefix).  For fb_step in sparse mode pass the
 * fb_sparse it will get; the larger of the SELECTED and COMPLEMENT plans is
 * returned.  Returns 0 on invalid arguments (see fb_last_error()). */
size_t fb_workspace_size(const fb_desc* d, const fb_sparse* sp);

/* Block-external partial (Core Mechanism: A_out and L_out = log Z_out) of every
 * block query over the prefix of its stream (or over the chunks `sp` picks),
 * split over the prefix and recombined by log-sum-exp weighting.
 * Writes o_ext [B][Hq][Lb][D] fp32 and lse_ext [B][Hq][Lb] fp32 (natural log;
 * -inf and a zero row for an empty prefix).  `ws` is scratch for the split
 * partials, at least fb_workspace_size(d, sp) bytes, 256-byte aligned. */
fb_status fb_prefix_attn(const fb_desc* d, const void* q_blk, const void* k_pre,
                         const void* v_pre, const fb_sparse* sp, float* o_ext,
                         float* lse_ext, void* ws, size_t ws_bytes, void* stream);

/* The two steps fb_prefix_attn is made of, callable on their own.
 * fb_prefix_partials: the split-KV pass only -- one normalised partial and its
 * natural-log LSE per (split, query head, block position), written to `ws` in
 * the layout fb_prefix_combine reads for the same (d, sp).
 * fb_prefix_combine: log-sum-exp combination of those partials (the merge
 * equation applied across the splits), optionally folding in one more partial
 * (extra_o [B][Hq][Lb][D], extra_lse [B][Hq][Lb], both or neither -- the
 * sparse variant's cached residual), into o_ext / lse_ext.  `sp` must be the
 * same fb_sparse (or NULL) as for the partials call.  o_ext and extra_o are
 * read and written as 16-byte vectors: both must be 16-byte aligned
 * (FB_ERR_ALIGN otherwise). */
fb_status fb_prefix_partials(const fb_desc* d, const void* q_blk, const void* k_pre,
                             const void* v_pre, const fb_sparse* sp, void* ws,
                             size_t ws_bytes, void* stream);
fb_status fb_prefix_combine(const fb_desc* d, const fb_sparse* sp, const float* extra_o,
                            const float* extra_lse, float* o_ext, float* lse_ext,
                            const void* ws, size_t ws_bytes, void* stream);

/* Block-internal attention (Core Mechanism: A_in over J_in, bidirectional)
 * of every block query over the block's own keys, merged with (o_ext, lse_ext)
 * by the merge equation when those are non-NULL (both or neither), written to
 * o [B][Lb][Hq][D] in the input dtype; lse_out (nullable) receives the merged
 * natural-log LSE [B][Hq][Lb]. */
fb_status fb_block_attn(const fb_desc* d, const void* q_blk, const void* k_blk,
                        const void* v_blk, const float* o_ext, const float* lse_ext,
                        void* o, float* lse_out, void* stream);

/* The merge equation on its own, row by row: rows x head_dim fp32 partials
 * (o_a, lse_a) and (o_b, lse_b) -> (o, lse).  o / lse may alias either input.
 * A row with both LSE = -inf yields o = 0, lse = -inf. */
fb_status fb_merge(int64_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                   const float* o_b, const float* lse_b, float* o, float* lse, void* stream);

/* One denoising step of the active block.
 * Refresh iff mode == FB_MODE_FULL, or force_refresh != 0, or step % r == 0
 * (step counts from 0 within the block, so step 0 always refreshes):
 *   dense (sp == NULL): refresh -> fb_prefix_attn into (o_ext_cache, lse_ext_cache);
 *                       every step -> fb_block_attn merged with the cache into o.
 *   sparse (sp != NULL, sp->mode ignored): refresh -> the COMPLEMENT partial into
 *                       (o_res_cache, lse_res_cache); every step -> the SELECTED
 *                       partial merged with the residual into (o_ext_cache,
 *                       lse_ext_cache), then the block partial merged into o.
 * A step that does not refresh reads caches written by an earlier refresh step of
 * the same block (same buffers); otherwise its result is undefined.  With the
 * environment variable FB_DEBUG=1 such a step first scans the cache it reads
 * (o/lse_ext_cache, or o/lse_res_cache in the sparse variant) for NaN, using the
 * first word of ws, waits for the answer on the stream, and returns FB_ERR_ARG
 * before launching anything else if it finds one (a debugging aid: it
 * synchronises the stream, so it is skipped while the stream is being
 * captured into a graph).
 * refreshed_out (host, nullable) receives 1 if this step refreshed.  Full mode
 * recomputes the prefix every step, i.e. the standard per-step attention over the
 * whole KV cache plus the block. */
fb_status fb_step(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk,
                  const void* k_pre, const void* v_pre, const fb_sparse* sp,
                  float* o_ext_cache, float* lse_ext_cache, float* o_res_cache,
                  float* lse_res_cache, void* o, float* lse_out, int32_t step,
                  int32_t refresh_period, int32_t mode, int32_t force_refresh,
                  int32_t* refreshed_out, void* ws, size_t ws_bytes, void* stream);

/* fb_step without a workspace, for callers that cannot allocate device memory:
 * code under graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments (less ws / ws_bytes), validation and results as
 * fb_step.  The split-KV partials go to a scratch array of
 * FB_NOALLOC_SCRATCH_BYTES that the library holds in the memory of every GPU
 * it runs on, from the first use until the process ends; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  The array
 * used is that of the calling thread's current device, which must be the
 * device of `stream`.  A shape whose fb_workspace_size(d, sp) exceeds the
 * scratch returns FB_ERR_WORKSPACE before anything is launched.  Every call on
 * one GPU shares that GPU's array and leaves its contents behind: calls that
 * overlap on one GPU (several streams or threads in flight at once) race and
 * give undefined results, so callers serialise them. */
#define FB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fb_status fb_step_noalloc(const fb_desc* d, const void* q_blk, const void* k_blk,
                          const void* v_blk, const void* k_pre, const void* v_pre,
                          const fb_sparse* sp, float* o_ext_cache, float* lse_ext_cache,
                          float* o_res_cache, float* lse_res_cache, void* o, float* lse_out,
                          int32_t step, int32_t refresh_period, int32_t mode,
                          int32_t force_refresh, int32_t* refreshed_out, void* stream);

/* Adaptive reuse (explainer page, "Adaptive Reuse Strategies"): instead of a
 * fixed refresh period, decide per step and per (stream, KV head) whether the
 * block-external partial is recomputed, entirely on the device.  A mask is
 * int32 [B][Hkv] in device memory, 1 = recompute at this step, 0 = reuse the
 * cached partial.  Step 0 of a block always sets every entry to 1.
 *
 * fb_refresh_mask_tau: threshold-based reuse.  M = the number of a stream's
 * block tokens whose K or V row (any KV head, any dim) differs from the
 * previous step's by more than eps (max-abs); every KV head of the stream is
 * recomputed iff M >= tau (the cache is reused while M < tau).  k_prev/v_prev
 * are the previous step's block K/V in the fb_desc block layout (not read at
 * step 0); after step 0 all four base pointers must be 16-byte aligned
 * (FB_ERR_ALIGN otherwise).  Writes count_out [B] (M; Lb at step 0) and mask_out [B][Hkv].  ws
 * holds B*Lb int32 flags (fb_workspace_size covers it).
 *
 * fb_refresh_mask_gamma: head-wise selection.  For each query head, the cosine
 * similarity (fp64 sums) of its block queries at the reference step (q_ref,
 * [B][Lb][Hq][D] contiguous, input dtype, caller-owned) and now (q_cur, fb_desc
 * q layout); 0 if a norm is 0.  KV head g is recomputed iff some query head of
 * its group has similarity <= gamma (it is reused only if all exceed gamma);
 * the group's q_ref rows then take the current queries.  Writes sim_out
 * [B][Hq] fp32 and mask_out.  At step 0 q_ref may hold anything.
 *
 * fb_step_masked: one dense step under a mask: the prefix pass and split
 * combine run only for the (stream, KV head) pairs the mask selects.  A
 * device-side unit plan (built from the mask in a small kernel, kept in ws)
 * lists those pairs and sizes their splits so that they alone fill the
 * grid; the other pairs get no work and their rows of o_ext_cache /
 * lse_ext_cache stay as they are.  Then the in-block pass merges with the
 * cache for every head into o.  The mask is read on the device, so no host
 * synchronisation is needed between the mask call and the step. */
fb_status fb_refresh_mask_tau(const fb_desc* d, const void* k_prev, const void* v_prev, const void* k_cur,
                              const void* v_cur, float eps, int32_t tau, int32_t step, int32_t* count_out,
                              int32_t* mask_out, void* ws, size_t ws_bytes, void* stream);
fb_status fb_refresh_mask_gamma(const fb_desc* d, const void* q_cur, void* q_ref, float gamma, int32_t step,
                                float* sim_out, int32_t* mask_out, void* stream);
fb_status fb_step_masked(const fb_desc* d, const void* q_blk, const void* k_blk, const void* v_blk,
                         const void* k_pre, const void* v_pre, const int32_t* mask, float* o_ext_cache,
                         float* lse_ext_cache, void* o, float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* Append the finalised block to the prefix KV cache (the cache the next
 * blocks read as J_out grows by each finalised block; explainer page, Problem
 * Statement).  Copies stream b's block K/V rows [Lb][Hkv][D] (fb_desc block
 * strides) into prefix rows dst_rows_dev[b] .. dst_rows_dev[b] + Lb - 1 of
 * k_pre / v_pre (fb_desc prefix strides, i.e. row r of KV head g at
 * r * pre_stride_t + g * pre_stride_h).  dst_rows_dev is int64 [B] in device
 * memory; the caller owns the capacity and afterwards describes the grown
 * prefix with new offsets.  Rows outside the written ones are not touched. */
fb_status fb_append_block(const fb_desc* d, const void* k_blk, const void* v_blk, void* k_pre, void* v_pre,
                          const int64_t* dst_rows_dev, void* stream);

/* Chunk selection for the sparse variant, on the device.  The pages pair
 * FlashBlock with a sparse-attention selector ("Compatibility with Sparse
 * Attention"; SparseD at 20-40% density) without stating the selector; this
 * one is the plainest block-level rule: each chunk of chunk_len prefix tokens
 * is represented by the mean of its keys (fp32), scored for a (stream, KV
 * head) by the largest dot product of that KV head's block queries with it,
 * and the k best chunks are kept (ties to the lower chunk index).  The chunk
 * list written is chunk_idx_out [B][Hkv][k] int32, ascending per (stream, KV
 * head) -- the fb_sparse chunk list.  Every stream needs at least k and at
 * most 16384 chunks; otherwise FB_ERR_ARG / FB_ERR_SHAPE.
 *
 * One-shot form: fb_select_chunks pools every chunk and selects.  ws holds
 * fb_select_chunks_ws(d, chunk_len) bytes, 256-byte aligned (pooled keys
 * [B][n_max][Hkv][D] fp32, then scores [B][Hkv][n_max] fp32, n_max = chunks
 * of the longest stream); fb_select_chunks_ws returns 0 on a bad desc. */
size_t fb_select_chunks_ws(const fb_desc* d, int32_t chunk_len);
fb_status fb_select_chunks(const fb_desc* d, const void* q_blk, const void* k_pre, int32_t chunk_len, int32_t k,
                           int32_t* chunk_idx_out, void* ws, size_t ws_bytes, void* stream);

/* Two-call form for an append-only prefix, whose chunk means do not change
 * once a chunk is full.  pooled: caller-owned fp32 [B][chunk_cap][Hkv][D]
 * (16-byte aligned), kept across blocks; chunk_cap >= chunks of the longest
 * stream.  fb_pool_chunk_keys (re)computes chunks first_chunk, first_chunk+1,
 * ... of every stream from k_pre (fb_desc prefix strides) and leaves lower
 * chunks untouched: after appending a block, first_chunk = the smallest old
 * stream length / chunk_len (rounded down) re-pools the partial last chunk
 * and pools the new ones.  fb_select_chunks_pooled scores and selects from
 * pooled; scores is caller-owned fp32 [B][Hkv][chunk_cap] scratch.  A
 * chunk_cap below the longest stream's chunk count is FB_ERR_ARG. */
fb_status fb_pool_chunk_keys(const fb_desc* d, const void* k_pre, int32_t chunk_len, int32_t chunk_cap,
                             int32_t first_chunk, float* pooled, void* stream);
fb_status fb_select_chunks_pooled(const fb_desc* d, const void* q_blk, const float* pooled, int32_t chunk_len,
                                  int32_t chunk_cap, int32_t k, float* scores, int32_t* chunk_idx_out,
                                  void* stream);

const char* fb_status_string(fb_status s);
const char* fb_last_error(void);
int32_t fb_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHBLOCK_H */
