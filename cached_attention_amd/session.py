"""Device buffers for one attention layer shape, driven through fb_step.

``AttentionStep`` allocates (with torch) the block-external cache, the sparse
residual cache, the split workspace and the output for one shape, and runs
denoising steps through the C ABI.  It adds no arithmetic of its own.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import flashblock as fbl

_DT = {"bf16": (fbl.FB_BF16, torch.bfloat16), "f32": (fbl.FB_F32, torch.float32)}


class AttentionStep:
    """Caches, workspace and outputs of one attention layer shape.

    dtype "bf16" or "f32"; ``prefix_offsets`` int [B+1] (stream b owns prefix
    rows off[b] .. off[b+1]-1); ``pre_strides`` (token stride, head stride) in
    elements of the prefix K/V, default token-major [T][Hkv][D].  With
    ``chunks`` (int32 [B][Hkv][k], ascending) the sparse variant runs: the
    residual of the unselected ``chunk_len``-token chunks is cached at refresh
    steps.  After a step, ``o`` [B][Lb][Hq][D] holds the output, ``lse``
    [B][Hq][Lb] its natural-log LSE, ``o_ext`` / ``lse_ext`` the block-external
    partial used (fp32).
    """

    def __init__(self, dtype: str, batch: int, hq: int, hkv: int, head_dim: int, block_len: int,
                 prefix_offsets: Sequence[int], device="cuda", chunks: Optional[torch.Tensor] = None,
                 chunk_len: int = 64, softmax_scale: float = 0.0, pre_strides=None):
        code, tdt = _DT[dtype]
        self.dtype, self.tdtype = dtype, tdt
        self.shape = (batch, hq, hkv, head_dim, block_len)
        self.offsets = np.asarray(prefix_offsets, dtype=np.int64)
        self.off_dev = torch.tensor(self.offsets, dtype=torch.int64, device=device)
        self.desc = fbl.Desc(code, batch, hq, hkv, head_dim, block_len, self.offsets, self.off_dev,
                             softmax_scale=softmax_scale, pre_strides=pre_strides)
        self.sparse = None
        if chunks is not None:
            self.chunks = chunks.to(device=device, dtype=torch.int32).contiguous()
            self.sparse = fbl.Sparse(self.chunks, int(self.chunks.shape[-1]), chunk_len)
        self.ws_bytes = fbl.fb_workspace_size(self.desc, self.sparse)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.o_ext = torch.zeros(batch, hq, block_len, head_dim, **f32)
        self.lse_ext = torch.full((batch, hq, block_len), float("-inf"), **f32)
        self.o_res = self.lse_res = None
        if self.sparse is not None:
            self.o_res = torch.zeros(batch, hq, block_len, head_dim, **f32)
            self.lse_res = torch.full((batch, hq, block_len), float("-inf"), **f32)
        self.o = torch.empty(batch, block_len, hq, head_dim, dtype=tdt, device=device)
        self.lse = torch.empty(batch, hq, block_len, **f32)

    def step(self, q, k, v, k_pre, v_pre, step: int, refresh_period: int = 1, mode: str = "cached",
             force_refresh: bool = False, want_lse: bool = True, stream=None) -> bool:
        """One denoising step through fb_step; returns whether it refreshed the cache.

        q [B][Lb][Hq][D], k / v [B][Lb][Hkv][D] (contiguous, this shape's dtype);
        ``step`` counts from 0 within the block; mode "cached" refreshes when
        step % refresh_period == 0 (or on ``force_refresh``), "full" every step.
        """
        m = fbl.FB_MODE_FULL if mode == "full" else fbl.FB_MODE_CACHED
        return fbl.fb_step(self.desc, q, k, v, k_pre, v_pre, self.sparse, self.o_ext, self.lse_ext,
                           self.o_res, self.lse_res, self.o, self.lse if want_lse else None, step,
                           refresh_period, m, force_refresh, self.ws, self.ws_bytes, stream)

    def step_policy(self, q, k, v, k_prev, v_prev, k_pre, v_pre, step: int, policy: str, tau: int = 0,
                    eps: float = 0.0, gamma: float = 0.0, want_lse: bool = True, stream=None) -> None:
        """One dense step under an adaptive reuse policy (dense prefix only).

        "tau": recompute a stream's block-external partials iff the number of
        block tokens whose K/V changed by more than eps since the previous step
        (k_prev, v_prev) reaches tau.  "gamma": recompute a KV head iff one of its
        query heads' block queries has cosine similarity <= gamma with the queries
        its cache was computed from.  The decision stays on the device:
        ``self.mask`` [B][Hkv] (1 = recomputed at this step), ``self.count`` [B]
        (tau) and ``self.sim`` [B][Hq] (gamma) hold the last step's values.
        """
        if self.sparse is not None:
            raise ValueError("adaptive reuse policies run on the dense prefix")
        b_n, hq, hkv, d, lb = self.shape
        if not hasattr(self, "mask"):
            dev = self.o.device
            self.mask = torch.zeros(b_n, hkv, dtype=torch.int32, device=dev)
            self.count = torch.zeros(b_n, dtype=torch.int32, device=dev)
            self.sim = torch.zeros(b_n, hq, dtype=torch.float32, device=dev)
            self.q_ref = torch.zeros(b_n, lb, hq, d, dtype=self.tdtype, device=dev)
        if policy == "tau":
            fbl.fb_refresh_mask_tau(self.desc, k_prev, v_prev, k, v, eps, tau, step, self.count, self.mask,
                                    self.ws, self.ws_bytes, stream)
        elif policy == "gamma":
            fbl.fb_refresh_mask_gamma(self.desc, q, self.q_ref, gamma, step, self.sim, self.mask, stream)
        else:
            raise ValueError(policy)
        fbl.fb_step_masked(self.desc, q, k, v, k_pre, v_pre, self.mask, self.o_ext, self.lse_ext, self.o,
                           self.lse if want_lse else None, self.ws, self.ws_bytes, stream)

    def prefix(self, q, k_pre, v_pre, chunk_mode: Optional[int] = None, stream=None) -> None:
        sp = None
        if chunk_mode is not None:
            sp = fbl.Sparse(self.chunks, int(self.chunks.shape[-1]), self.sparse.c.chunk_len, chunk_mode)
        fbl.fb_prefix_attn(self.desc, q, k_pre, v_pre, sp, self.o_ext, self.lse_ext, self.ws, self.ws_bytes,
                           stream)

    def block(self, q, k, v, merge: bool = True, stream=None) -> None:
        fbl.fb_block_attn(self.desc, q, k, v, self.o_ext if merge else None, self.lse_ext if merge else None,
                          self.o, self.lse, stream)
