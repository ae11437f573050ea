"""fp64 definitions of the FlashBlock attention step (test infrastructure only).

Every function here is written for a reader checking it against the FlashBlock
pages by eye: NumPy float64, one head at a time, no tiling, no fusion, no
reordering beyond what the definitions state.  A matmul, an exp and a max are
the only library primitives used.

Notation (FlashBlock explainer page, Technical Summary section 2, "Core
Mechanism"): the keys a block's queries see split into J_in (the block's own
tokens) and J_out (everything outside the block, i.e. the KV cache of earlier,
finalised blocks).  A is an attention output normalised over its key set and
L = log Z its log-normaliser; two such partials combine with the page's merge
equation.

Readings of points the pages leave open (all taken as the plainest one):
  * softmax scale 1/sqrt(D) unless the caller gives another;
  * L is a natural log (the merge equation weighs partials by e^(L - m));
  * A is normalised (sum_t p_t v_t / Z), which is what makes the merge exact;
  * inside the block attention is bidirectional (no mask), and the block sees
    the whole prefix;
  * grouped-query attention: query head h reads KV head h // (Hq / Hkv);
  * an empty key set has A = 0 and L = -inf, and merging with it returns the
    other partial unchanged;
  * the cache is refreshed at step s of a block iff s mod r == 0 (step 0 always
    refreshes), or on every step in full-recompute mode.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# One head: partial attention and the merge
# ---------------------------------------------------------------------------

def partial_attention(q, k, v, scale: float):
    """Attention of query rows over one key set: (A, L).

    q: [n, D]; k, v: [m, D].  For each row i:
        s_t = scale * <q_i, k_t>,   mx = max_t s_t,   Z = sum_t exp(s_t - mx),
        A_i = sum_t exp(s_t - mx) v_t / Z,   L_i = mx + log Z.
    This is the block-external (or block-internal) attention output and its
    log-normaliser L = log Z of the Core Mechanism section.  An empty key set
    gives A = 0 and L = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    dv = v.shape[1] if v.ndim == 2 else q.shape[1]
    if k.shape[0] == 0:
        return np.zeros((n, dv)), np.full(n, NEG_INF)
    s = scale * (q @ k.T)
    mx = s.max(axis=1)
    p = np.exp(s - mx[:, None])
    z = p.sum(axis=1)
    a = (p @ v) / z[:, None]
    return a, mx + np.log(z)


def merge(a_out, l_out, a_in, l_in):
    """The merge equation of the Core Mechanism section, row by row.

    m = max(L_out, L_in);
    A = (e^(L_out - m) A_out + e^(L_in - m) A_in) / (e^(L_out - m) + e^(L_in - m)).
    The merged log-normaliser (implied, not printed on the page) is
    L = m + log(e^(L_out - m) + e^(L_in - m)).  When one side is empty
    (L = -inf) its weight is 0; when both are, A = 0 and L = -inf.
    """
    a_out = np.asarray(a_out, dtype=np.float64)
    a_in = np.asarray(a_in, dtype=np.float64)
    l_out = np.asarray(l_out, dtype=np.float64)
    l_in = np.asarray(l_in, dtype=np.float64)
    m = np.maximum(l_out, l_in)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    w_out = np.exp(l_out - m_safe)
    w_in = np.exp(l_in - m_safe)
    den = w_out + w_in
    den_safe = np.where(both_empty, 1.0, den)
    a = (w_out[..., None] * a_out + w_in[..., None] * a_in) / den_safe[..., None]
    lse = m_safe + np.log(den_safe)
    a = np.where(both_empty[..., None], 0.0, a)
    lse = np.where(both_empty, NEG_INF, lse)
    return a, lse


# ---------------------------------------------------------------------------
# The library's layouts
#   Q_blk, O      [B][Lb][Hq][D]
#   K_blk, V_blk  [B][Lb][Hkv][D]
#   K_pre, V_pre  [T][Hkv][D] packed; stream b owns rows offsets[b]..offsets[b+1]
#   O_ext, LSE    [B][Hq][Lb][D] and [B][Hq][Lb]
# ---------------------------------------------------------------------------

def kv_group(h: int, hq: int, hkv: int) -> int:
    """KV head read by query head h (contiguous groups of Hq/Hkv query heads)."""
    return h // (hq // hkv)


def prefix_token_sets(lp: int, chunks=None, chunk_len: int = 64, mode: str = "all"):
    """Token indices (within one stream's prefix) that a partial attends to.

    mode "all": the whole prefix.  For the sparse variant (Adaptive Reuse
    Strategies, "Compatibility with Sparse Attention"): "selected" is the union
    of the listed chunks [c*chunk_len, (c+1)*chunk_len) clipped to the prefix,
    and "complement" is every other prefix token -- the unselected keys whose
    contribution the page caches as the residual.
    """
    if mode == "all":
        return np.arange(lp)
    sel = np.zeros(lp, dtype=bool)
    for c in np.asarray(chunks).tolist():
        sel[c * chunk_len: min((c + 1) * chunk_len, lp)] = True
    if mode == "selected":
        return np.nonzero(sel)[0]
    if mode == "complement":
        return np.nonzero(~sel)[0]
    raise ValueError(mode)


def prefix_partial(q_blk, k_pre, v_pre, offsets, scale: float,
                   chunks=None, chunk_len: int = 64, mode: str = "all"):
    """Block-external partial (A_out, L_out) for every stream, query head and row.

    Returns O [B][Hq][Lb][D] and L [B][Hq][Lb].
    """
    b_n, lb, hq, d = q_blk.shape
    hkv = k_pre.shape[1]
    o = np.zeros((b_n, hq, lb, d))
    lse = np.zeros((b_n, hq, lb))
    for b in range(b_n):
        t0, t1 = int(offsets[b]), int(offsets[b + 1])
        for h in range(hq):
            g = kv_group(h, hq, hkv)
            idx = prefix_token_sets(t1 - t0, None if chunks is None else chunks[b][g],
                                    chunk_len, mode)
            k = k_pre[t0:t1, g, :][idx]
            v = v_pre[t0:t1, g, :][idx]
            o[b, h], lse[b, h] = partial_attention(q_blk[b, :, h, :], k, v, scale)
    return o, lse


def block_partial(q_blk, k_blk, v_blk, scale: float):
    """Block-internal partial (A_in, L_in): every block query over every block key."""
    b_n, lb, hq, d = q_blk.shape
    hkv = k_blk.shape[2]
    o = np.zeros((b_n, hq, lb, d))
    lse = np.zeros((b_n, hq, lb))
    for b in range(b_n):
        for h in range(hq):
            g = kv_group(h, hq, hkv)
            o[b, h], lse[b, h] = partial_attention(q_blk[b, :, h, :], k_blk[b, :, g, :],
                                                   v_blk[b, :, g, :], scale)
    return o, lse


def merge_outputs(o_a, l_a, o_b, l_b):
    """Merge two cache-layout partials; returns (O [B][Hq][Lb][D], L [B][Hq][Lb])."""
    return merge(o_a, l_a, o_b, l_b)


def to_output_layout(o_cache_layout):
    """[B][Hq][Lb][D] -> [B][Lb][Hq][D]."""
    return np.ascontiguousarray(np.transpose(o_cache_layout, (0, 2, 1, 3)))


def full_step(q_blk, k_blk, v_blk, k_pre, v_pre, offsets, scale: float):
    """Exact attention of every block query over prefix + block keys.

    Computed directly over the concatenated key set J_out + J_in, never through
    the merge, so that it can check the merge.  Returns O [B][Lb][Hq][D] and
    L [B][Hq][Lb].
    """
    b_n, lb, hq, d = q_blk.shape
    hkv = k_blk.shape[2]
    o = np.zeros((b_n, hq, lb, d))
    lse = np.zeros((b_n, hq, lb))
    for b in range(b_n):
        t0, t1 = int(offsets[b]), int(offsets[b + 1])
        for h in range(hq):
            g = kv_group(h, hq, hkv)
            k = np.concatenate([k_pre[t0:t1, g, :], k_blk[b, :, g, :]], axis=0)
            v = np.concatenate([v_pre[t0:t1, g, :], v_blk[b, :, g, :]], axis=0)
            o[b, h], lse[b, h] = partial_attention(q_blk[b, :, h, :], k, v, scale)
    return to_output_layout(o), lse


# ---------------------------------------------------------------------------
# A block of denoising steps: cached block-external attention vs full recompute
# ---------------------------------------------------------------------------

@dataclass
class BlockResult:
    out: List[np.ndarray] = field(default_factory=list)       # per step O [B][Lb][Hq][D]
    lse: List[np.ndarray] = field(default_factory=list)       # per step L [B][Hq][Lb]
    refreshed: List[bool] = field(default_factory=list)
    o_ext: List[np.ndarray] = field(default_factory=list)     # cache as used at each step
    lse_ext: List[np.ndarray] = field(default_factory=list)


def refresh_due(step: int, r: int, mode: str) -> bool:
    """Refresh schedule: every step in full mode, else iff step mod r == 0."""
    if r < 1 or step < 0:
        raise ValueError("r >= 1 and step >= 0 required")
    return mode == "full" or step % r == 0


def run_block(k_pre, v_pre, offsets, q_steps, k_steps, v_steps, scale: float,
              r: int = 1, mode: str = "cached", chunks=None, chunk_len: int = 64):
    """Outputs of one block's denoising steps.

    mode "full": every step is the exact attention over prefix + block
    (``full_step``), the standard block-diffusion step that recomputes over
    the whole growing KV cache.

    mode "cached" (the Core Mechanism section): at a refresh step the
    block-external partial (A_out, L_out) of that step's queries is computed
    and kept; every step computes the block-internal partial of its own
    queries and merges it with the kept (A_out, L_out).

    With ``chunks`` (int [B][Hkv][k]) the sparse variant of Adaptive Reuse
    Strategies ("Compatibility with Sparse Attention") runs instead: the
    refresh step keeps the partial over the unselected prefix chunks as the
    residual, and every step merges residual, a fresh partial over the selected
    chunks, and the block-internal partial.
    """
    res = BlockResult()
    cache_o = cache_l = None
    for s in range(len(q_steps)):
        q, kb, vb = q_steps[s], k_steps[s], v_steps[s]
        if mode == "full":
            o, lse = full_step(q, kb, vb, k_pre, v_pre, offsets, scale)
            res.out.append(o)
            res.lse.append(lse)
            res.refreshed.append(True)
            continue
        refresh = refresh_due(s, r, mode)
        if refresh:
            if chunks is None:
                cache_o, cache_l = prefix_partial(q, k_pre, v_pre, offsets, scale)
            else:
                cache_o, cache_l = prefix_partial(q, k_pre, v_pre, offsets, scale,
                                                  chunks, chunk_len, "complement")
        if chunks is None:
            ext_o, ext_l = cache_o, cache_l
        else:
            sel_o, sel_l = prefix_partial(q, k_pre, v_pre, offsets, scale,
                                          chunks, chunk_len, "selected")
            ext_o, ext_l = merge(cache_o, cache_l, sel_o, sel_l)
        in_o, in_l = block_partial(q, kb, vb, scale)
        o, lse = merge(ext_o, ext_l, in_o, in_l)
        res.out.append(to_output_layout(o))
        res.lse.append(lse)
        res.refreshed.append(refresh)
        res.o_ext.append(ext_o)
        res.lse_ext.append(ext_l)
    return res


def sparse_only_step(q_blk, k_blk, v_blk, k_pre, v_pre, offsets, scale, chunks, chunk_len=64):
    """Context baseline: sparse attention without the cached residual.

    The keys are the selected chunks of the prefix (per stream and KV head,
    clipped to the prefix) and the block's own keys; the unselected chunks,
    whose contribution the sparse variant keeps as its residual, are left out
    entirely.  Returns O [B][Lb][Hq][D]."""
    sel_o, sel_l = prefix_partial(q_blk, k_pre, v_pre, offsets, scale, chunks, chunk_len, "selected")
    in_o, in_l = block_partial(q_blk, k_blk, v_blk, scale)
    o, _ = merge(sel_o, sel_l, in_o, in_l)
    return to_output_layout(o)


def grow_prefix(k_pre, v_pre, offsets, k_last, v_last):
    """Append the block's final-step K/V to each stream's prefix (the block is
    finalised and joins the KV cache of earlier blocks for the next block).

    k_last, v_last: [B][Lb][Hkv][D].  Returns new (k_pre, v_pre, offsets).
    """
    b_n = k_last.shape[0]
    ks, vs = [], []
    new_off = np.zeros(b_n + 1, dtype=np.int64)
    for b in range(b_n):
        t0, t1 = int(offsets[b]), int(offsets[b + 1])
        ks.append(k_pre[t0:t1])
        ks.append(k_last[b])
        vs.append(v_pre[t0:t1])
        vs.append(v_last[b])
        new_off[b + 1] = new_off[b] + (t1 - t0) + k_last.shape[1]
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0), new_off


def append_block_rows(k_pre, v_pre, k_last, v_last, dst_rows):
    """Write each stream's finalised block K/V into given prefix rows.

    Once a block is final it joins the growing KV cache that the next blocks'
    queries read as J_out (explainer page, Problem Statement: block-wise
    causal inference over a growing KV cache).  Stream b's Lb rows go to
    prefix rows dst_rows[b] ..
    dst_rows[b] + Lb - 1 (all KV heads).  Returns new arrays; the inputs are
    not modified.
    """
    k_new = np.array(k_pre, copy=True)
    v_new = np.array(v_pre, copy=True)
    lb = k_last.shape[1]
    for b in range(k_last.shape[0]):
        r0 = int(dst_rows[b])
        k_new[r0:r0 + lb] = k_last[b]
        v_new[r0:r0 + lb] = v_last[b]
    return k_new, v_new
