"""Seeded synthetic inputs for the FlashBlock attention step.

This module only draws and rounds numbers; it holds none of the attention
arithmetic, so the HIP path and the fp64 oracle can both be fed from it.

Recipe (the FlashBlock pages name their workloads -- Trado-8B/4B text models and
the LongLive-1.3B video model, Technical Summary section 4 -- but no shapes and
no activations; these synthetic shapes stand in for them):

* one ``numpy.random.default_rng(seed)`` (PCG64) stream per workload;
* draw order: [ragged prefix lengths], prefix K, prefix V, then for every block
  Q0, K0, V0 followed by, per later step s = 1..S-1, the noise for Q, K, V;
* values are ``value_scale * N(0, 1)`` drawn in float32;
* block tokens move as a random walk across denoising steps:
  ``X_s = round(X_{s-1} + sigma * eps_s)`` with fresh ``eps_s`` per step; the
  prefix is fixed within a block;
* bf16 workloads round every value to bfloat16 with round-to-nearest-even, so
  both sides see exactly the values the GPU stores.

Arrays are returned as float32 holding exactly representable values; the
layouts are the library's: Q/K/V of the block ``[S][B][Lb][H][D]`` and the
packed ragged prefix ``[T][Hkv][D]`` with int64 stream offsets ``[B+1]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "round_bf16",
    "bf16_bits",
    "make_prefix",
    "make_block_steps",
    "make_chunk_selection",
    "ci_version",
]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    nan = np.isnan(x)
    out = rounded.view(np.float32).copy()
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns of float32 values already rounded to bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    batch: int
    hq: int
    hkv: int
    head_dim: int
    block_len: int
    prefix_len: int            # mean prefix length per stream at the first block
    steps: int                 # denoising steps per block
    value_scale: float
    drift_sigma: float
    refresh_periods: tuple = (1,)
    n_blocks: int = 1
    ragged: float = 0.0        # +-fraction of per-stream prefix length jitter
    sparse_keep: float = 0.0   # fraction of 64-token prefix chunks kept (0: dense only)
    chunk_len: int = 64
    seed: int = 20260
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.hq // self.hkv


WORKLOADS = {
    # tiny fp32 single layer: the small case the oracle finishes at once
    "tiny_f32": Workload("tiny_f32", "f32", 1, 4, 4, 64, 16, 256, 4, 1.0, 0.1,
                         refresh_periods=(1, 2, 4), seed=20260),
    # LLaDA-8B-like text layer, MHA 32 heads, block 32, prefix sweep
    "text_mha_4k": Workload("text_mha_4k", "bf16", 1, 32, 32, 128, 32, 4096, 8, 0.5, 0.05,
                            refresh_periods=(1, 4, 8), seed=20261),
    "text_mha_16k": Workload("text_mha_16k", "bf16", 1, 32, 32, 128, 32, 16384, 8, 0.5, 0.05,
                             refresh_periods=(1, 4, 8), seed=20261),
    "text_mha_32k": Workload("text_mha_32k", "bf16", 1, 32, 32, 128, 32, 32768, 8, 0.5, 0.05,
                             refresh_periods=(1, 4, 8), seed=20261),
    # long-context text with GQA 32/8, block 64, 128K prefix (+ 10% chunk-sparse variant)
    "text_gqa_128k": Workload("text_gqa_128k", "bf16", 1, 32, 8, 128, 64, 131072, 8, 0.5, 0.05,
                              refresh_periods=(1, 8), sparse_keep=0.10, seed=20262),
    # video block diffusion: 12 heads, one 1560-token latent frame per block,
    # 20-frame prefix growing by one frame per block
    "video_1560": Workload("video_1560", "bf16", 1, 12, 12, 128, 1560, 31200, 4, 1.0, 0.1,
                           refresh_periods=(1, 4), n_blocks=4, seed=20263),
    # 8 independent streams, GQA 32/8, block 32, ragged ~64K prefixes
    "batched_64k": Workload("batched_64k", "bf16", 8, 32, 8, 128, 32, 65536, 8, 0.5, 0.05,
                            refresh_periods=(1, 2, 8), ragged=0.25, seed=20264),
}


def ci_version(w: Workload, prefix_len: int, block_len: Optional[int] = None,
               hq: Optional[int] = None, hkv: Optional[int] = None,
               batch: Optional[int] = None, n_blocks: Optional[int] = None) -> Workload:
    """A scaled-down copy of a workload (same dtype, value law and structure)."""
    kw = dict(prefix_len=prefix_len, name=w.name + f"_ci{prefix_len}")
    if block_len is not None:
        kw["block_len"] = block_len
    if hq is not None:
        kw["hq"] = hq
    if hkv is not None:
        kw["hkv"] = hkv
    if batch is not None:
        kw["batch"] = batch
    if n_blocks is not None:
        kw["n_blocks"] = n_blocks
    return replace(w, **kw)


def _draw(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return round_bf16(x) if dtype == "bf16" else x


def _prefix_lengths(w: Workload, rng: np.random.Generator) -> List[int]:
    if w.ragged <= 0.0 or w.batch == 1:
        return [w.prefix_len] * w.batch
    u = rng.uniform(-w.ragged, w.ragged, size=w.batch)
    return [int(np.round(w.prefix_len * (1.0 + ub))) for ub in u]  # numpy rounds half to even


@dataclass
class Prefix:
    k: np.ndarray              # [T][Hkv][D] float32
    v: np.ndarray              # [T][Hkv][D] float32
    offsets: np.ndarray        # int64 [B+1]

    @property
    def lengths(self) -> List[int]:
        return [int(self.offsets[b + 1] - self.offsets[b]) for b in range(len(self.offsets) - 1)]


def make_prefix(w: Workload, rng: np.random.Generator) -> Prefix:
    """Draws the prefix lengths (ragged workloads), then prefix K, then prefix V."""
    lens = _prefix_lengths(w, rng)
    offsets = np.zeros(w.batch + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    t = int(offsets[-1])
    k = _draw(rng, (t, w.hkv, w.head_dim), w.value_scale, w.dtype)
    v = _draw(rng, (t, w.hkv, w.head_dim), w.value_scale, w.dtype)
    return Prefix(k, v, offsets)


@dataclass
class BlockSteps:
    q: np.ndarray              # [S][B][Lb][Hq][D]
    k: np.ndarray              # [S][B][Lb][Hkv][D]
    v: np.ndarray              # [S][B][Lb][Hkv][D]


def make_block_steps(w: Workload, rng: np.random.Generator) -> BlockSteps:
    """Step-0 block tokens, then the per-step random-walk noise for Q, K and V."""
    qs = (w.batch, w.block_len, w.hq, w.head_dim)
    ks = (w.batch, w.block_len, w.hkv, w.head_dim)
    q = np.empty((w.steps,) + qs, dtype=np.float32)
    k = np.empty((w.steps,) + ks, dtype=np.float32)
    v = np.empty((w.steps,) + ks, dtype=np.float32)
    q[0] = _draw(rng, qs, w.value_scale, w.dtype)
    k[0] = _draw(rng, ks, w.value_scale, w.dtype)
    v[0] = _draw(rng, ks, w.value_scale, w.dtype)
    for s in range(1, w.steps):
        for arr, shape in ((q, qs), (k, ks), (v, ks)):
            eps = rng.standard_normal(size=shape, dtype=np.float32)
            nxt = arr[s - 1] + np.float32(w.drift_sigma) * eps
            arr[s] = round_bf16(nxt) if w.dtype == "bf16" else nxt
    return BlockSteps(q, k, v)


def make_block_steps_decoding(w: Workload, rng: np.random.Generator, head_spread: float = 0.0,
                              reveal: bool = True) -> BlockSteps:
    """Block steps that imitate progressive unmasking, for the adaptive reuse policies.

    Step 0 draws every token as in ``make_block_steps``.  The block's Lb tokens
    are then revealed over steps 1 .. S-1 in seeded, uneven batches (a
    multinomial split): a revealed token's Q, K and V rows are redrawn once
    (an abrupt update), every other token takes the random-walk step.  With
    ``head_spread`` > 0, query head h drifts with sigma * u_h, u_h ~ U[1 -
    head_spread, 1 + head_spread] (seeded), so heads vary across steps unevenly
    (the video case of head-wise selection); ``reveal=False`` keeps only the
    drift (every token changes a little, none abruptly).  Draw order: reveal counts,
    per-head factors, step 0 tokens, then per step: the revealed set, fresh
    rows, and the noise for Q, K, V.
    """
    steps, lb = w.steps, w.block_len
    counts = rng.multinomial(lb, [1.0 / max(1, steps - 1)] * max(1, steps - 1)) if steps > 1 else np.zeros(0, int)
    u = (rng.uniform(1.0 - head_spread, 1.0 + head_spread, size=w.hq).astype(np.float32)
         if head_spread > 0 else np.ones(w.hq, dtype=np.float32))
    qs = (w.batch, lb, w.hq, w.head_dim)
    ks = (w.batch, lb, w.hkv, w.head_dim)
    q = np.empty((steps,) + qs, dtype=np.float32)
    k = np.empty((steps,) + ks, dtype=np.float32)
    v = np.empty((steps,) + ks, dtype=np.float32)
    q[0] = _draw(rng, qs, w.value_scale, w.dtype)
    k[0] = _draw(rng, ks, w.value_scale, w.dtype)
    v[0] = _draw(rng, ks, w.value_scale, w.dtype)
    hidden = np.arange(lb)
    sig = np.float32(w.drift_sigma)
    for s in range(1, steps):
        n = int(counts[s - 1]) if reveal else 0
        shown = rng.choice(hidden, size=min(n, len(hidden)), replace=False) if n > 0 else np.zeros(0, int)
        hidden = np.setdiff1d(hidden, shown)
        fq, fk, fv = (_draw(rng, (w.batch, len(shown)) + sh[2:], w.value_scale, w.dtype) for sh in (qs, ks, ks))
        eq = rng.standard_normal(size=qs, dtype=np.float32) * (sig * u)[None, None, :, None]
        ek = rng.standard_normal(size=ks, dtype=np.float32) * sig
        ev = rng.standard_normal(size=ks, dtype=np.float32) * sig
        for arr, eps_, fresh in ((q, eq, fq), (k, ek, fk), (v, ev, fv)):
            nxt = arr[s - 1] + eps_
            nxt[:, shown] = fresh
            arr[s] = round_bf16(nxt) if w.dtype == "bf16" else nxt
    return BlockSteps(q, k, v)


def make_chunk_selection(w: Workload, prefix_lengths: List[int], seed_offset: int = 1000) -> np.ndarray:
    """Seeded stand-in for a sparse-attention chunk selector.

    For every (stream, KV head) keeps ceil(keep * n_chunks) of the 64-token prefix
    chunks, chosen uniformly without replacement and sorted ascending.  Returns
    int32 ``[B][Hkv][k]``; k is taken from the shortest stream so the array is
    rectangular.
    """
    rng = np.random.default_rng(w.seed + seed_offset)
    nchunks = [(lp + w.chunk_len - 1) // w.chunk_len for lp in prefix_lengths]
    kmin = min(int(np.ceil(w.sparse_keep * n)) for n in nchunks)
    out = np.empty((w.batch, w.hkv, kmin), dtype=np.int32)
    for b in range(w.batch):
        for g in range(w.hkv):
            sel = rng.choice(nchunks[b], size=kmin, replace=False)
            out[b, g] = np.sort(sel).astype(np.int32)
    return out


def make_inputs(w: Workload):
    """Prefix and every block's steps, drawn in the recipe's order from one stream."""
    rng = np.random.default_rng(w.seed)
    prefix = make_prefix(w, rng)
    blocks = [make_block_steps(w, rng) for _ in range(w.n_blocks)]
    return prefix, blocks
