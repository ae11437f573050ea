"""fp64 definitions of FlashBlock's adaptive reuse policies (test infrastructure only).

Source: the FlashBlock explainer page, Technical Summary, "Adaptive Reuse
Strategies".  Two policies decide, per denoising step, whether the cached
block-external partial is reused or recomputed:

  * threshold-based reuse: a threshold tau on the number M^{s+1} of block
    tokens updated at the step; the cache is reused while M^{s+1} < tau and
    recomputed otherwise;
  * head-wise selection (video): a similarity is estimated per attention head;
    only heads whose similarity exceeds gamma reuse the cache.

Readings of what the page leaves open (plainest choices):
  * "updated token": a block token whose K or V row (any KV head, any dim)
    differs by more than eps (max-abs) from the previous step's; M is counted
    per stream and the decision is per stream;
  * "similarity of a head": the cosine similarity between the head's block
    queries (flattened over positions and dims) at the step its cache was last
    computed and at the current step; a head refreshes iff the similarity is
    <= gamma (reuse iff it exceeds gamma), or if either query norm is zero;
  * the prefix pass works per KV head, so a KV head is recomputed iff any of
    its query heads needs it (for the MHA video workload the two coincide);
  * step 0 of a block always computes the cache (there is none yet);
  * after a KV head is recomputed its reference queries are the current ones.

Masks are int arrays [B][Hkv]: 1 = recompute the block-external partial of
this (stream, KV head) at this step, 0 = reuse the cached one.

The module also holds the chunk selection of the sparse variant (pooled chunk
keys, max query score, top-k; its own section below, with its readings).
"""
from __future__ import annotations

import numpy as np

from .attention import (BlockResult, block_partial, kv_group, merge, prefix_partial,
                        to_output_layout)


def updated_tokens(k_prev, v_prev, k_cur, v_cur, eps: float):
    """M per stream: block tokens whose K or V row changed by more than eps.

    k_*, v_*: [B][Lb][Hkv][D].  Returns int64 [B].
    """
    dk = np.abs(np.asarray(k_cur, np.float64) - np.asarray(k_prev, np.float64)).max(axis=(2, 3))
    dv = np.abs(np.asarray(v_cur, np.float64) - np.asarray(v_prev, np.float64)).max(axis=(2, 3))
    changed = (dk > eps) | (dv > eps)
    return changed.sum(axis=1).astype(np.int64)


def tau_mask(m_count, tau: int, step: int, hkv: int):
    """Recompute a stream's partials iff M >= tau (reuse iff M < tau); step 0 always."""
    b_n = len(m_count)
    mask = np.zeros((b_n, hkv), dtype=np.int32)
    for b in range(b_n):
        if step == 0 or m_count[b] >= tau:
            mask[b, :] = 1
    return mask


def head_similarity(q_ref, q_cur):
    """Cosine similarity per (stream, query head) of the block queries.

    q_ref, q_cur: [B][Lb][Hq][D].  Returns float64 [B][Hq]; 0 where a norm is 0.
    """
    a = np.asarray(q_ref, np.float64)
    c = np.asarray(q_cur, np.float64)
    b_n, _, hq, _ = a.shape
    sim = np.zeros((b_n, hq))
    for b in range(b_n):
        for h in range(hq):
            x = a[b, :, h, :].ravel()
            y = c[b, :, h, :].ravel()
            nx, ny = float(np.dot(x, x)), float(np.dot(y, y))
            sim[b, h] = float(np.dot(x, y)) / np.sqrt(nx * ny) if nx > 0 and ny > 0 else 0.0
    return sim


def gamma_mask(sim, gamma: float, step: int, hq: int, hkv: int):
    """Recompute KV head g iff some query head of its group has similarity <= gamma."""
    b_n = sim.shape[0]
    mask = np.zeros((b_n, hkv), dtype=np.int32)
    for b in range(b_n):
        for h in range(hq):
            if step == 0 or not (sim[b, h] > gamma):
                mask[b, kv_group(h, hq, hkv)] = 1
    return mask


def run_block_policy(k_pre, v_pre, offsets, q_steps, k_steps, v_steps, scale: float, policy: str,
                     tau: int = 0, eps: float = 0.0, gamma: float = 0.0, masks=None):
    """One block's steps with per-(stream, KV head) recompute decisions.

    policy "tau" or "gamma" derives the masks as above; policy "given" takes
    ``masks`` (one [B][Hkv] array per step).  At each step the block-external
    partial of every masked (stream, KV head) is recomputed from that step's
    queries and kept; every other one is reused from its last computation; the
    block-internal partial is always fresh and merged in.

    Returns a BlockResult with an extra list ``masks`` (the masks used) and,
    for "tau", ``counts`` (M per stream and step), for "gamma", ``sims``.
    """
    b_n, lb, hq, d = q_steps[0].shape
    hkv = k_steps[0].shape[2]
    res = BlockResult()
    res.masks, res.counts, res.sims = [], [], []
    cache_o = np.zeros((b_n, hq, lb, d))
    cache_l = np.full((b_n, hq, lb), -np.inf)
    q_ref = None
    for s in range(len(q_steps)):
        q, kb, vb = q_steps[s], k_steps[s], v_steps[s]
        if policy == "tau":
            m = (updated_tokens(k_steps[s - 1], v_steps[s - 1], kb, vb, eps) if s > 0
                 else np.full(b_n, lb, dtype=np.int64))
            mask = tau_mask(m, tau, s, hkv)
            res.counts.append(m)
        elif policy == "gamma":
            sim = head_similarity(q_ref, q) if s > 0 else np.zeros((b_n, hq))
            mask = gamma_mask(sim, gamma, s, hq, hkv)
            res.sims.append(sim)
            if q_ref is None:
                q_ref = np.array(q, dtype=np.float64)
            for b in range(b_n):
                for h in range(hq):
                    if mask[b, kv_group(h, hq, hkv)]:
                        q_ref[b, :, h, :] = q[b, :, h, :]
        elif policy == "given":
            mask = np.asarray(masks[s], dtype=np.int32)
        else:
            raise ValueError(policy)
        if mask.any():
            fresh_o, fresh_l = prefix_partial(q, k_pre, v_pre, offsets, scale)
            for b in range(b_n):
                for h in range(hq):
                    if mask[b, kv_group(h, hq, hkv)]:
                        cache_o[b, h] = fresh_o[b, h]
                        cache_l[b, h] = fresh_l[b, h]
        in_o, in_l = block_partial(q, kb, vb, scale)
        o, lse = merge(cache_o, cache_l, in_o, in_l)
        res.out.append(to_output_layout(o))
        res.lse.append(lse)
        res.refreshed.append(bool(mask.any()))
        res.o_ext.append(cache_o.copy())
        res.lse_ext.append(cache_l.copy())
        res.masks.append(mask)
    return res


# ---------------------------------------------------------------------------
# Chunk selection for the sparse variant
# ---------------------------------------------------------------------------
#
# The pages combine FlashBlock with a sparse-attention selector (SparseD at
# 20-40% density; "Compatibility with Sparse Attention") without stating the
# selector.  Reading taken here (the plainest block-level rule): a chunk of
# chunk_len prefix tokens is represented by the mean of its keys; its score
# for a (stream, KV head) is the largest dot product any query of the KV
# head's group has with that pooled key; the k best chunks are kept, ties
# going to the lower chunk index, listed ascending.

def pooled_chunk_keys(k_pre, offsets, chunk_len: int = 64):
    """Mean key per chunk: list over streams of [n_chunks_b][Hkv][D] (fp64)."""
    out = []
    for b in range(len(offsets) - 1):
        t0, t1 = int(offsets[b]), int(offsets[b + 1])
        n = -(-(t1 - t0) // chunk_len)
        pk = np.zeros((n, k_pre.shape[1], k_pre.shape[2]))
        for c in range(n):
            a, z = t0 + c * chunk_len, min(t0 + (c + 1) * chunk_len, t1)
            pk[c] = np.asarray(k_pre[a:z], np.float64).mean(axis=0)
        out.append(pk)
    return out


def chunk_scores(q_blk, pooled):
    """score[b][g][c] = max over the group's block queries of q . pooled key."""
    b_n, lb, hq, d = q_blk.shape
    hkv = pooled[0].shape[1] if len(pooled[0]) else 1
    scores = []
    for b in range(b_n):
        n = pooled[b].shape[0]
        sb = np.full((hkv, n), -np.inf)
        for g in range(hkv):
            qs = np.concatenate([np.asarray(q_blk[b, :, h, :], np.float64)
                                 for h in range(hq) if kv_group(h, hq, hkv) == g], axis=0)
            if n:
                sb[g] = (qs @ pooled[b][:, g, :].T).max(axis=0)
        scores.append(sb)
    return scores


def select_chunks(q_blk, k_pre, offsets, k: int, chunk_len: int = 64):
    """Top-k chunk indices per (stream, KV head), ascending: int32 [B][Hkv][k]."""
    pooled = pooled_chunk_keys(k_pre, offsets, chunk_len)
    scores = chunk_scores(q_blk, pooled)
    b_n = len(scores)
    hkv = scores[0].shape[0]
    idx = np.zeros((b_n, hkv, k), dtype=np.int32)
    for b in range(b_n):
        for g in range(hkv):
            s = scores[b][g]
            order = sorted(range(len(s)), key=lambda c: (-s[c], c))   # best first, ties: lower index
            idx[b, g] = np.sort(np.array(order[:k], dtype=np.int32))
    return idx
