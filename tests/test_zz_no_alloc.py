"""fb_step_noalloc: fb_step with the library's per-GPU scratch array instead
of a caller workspace (for callers that cannot allocate).

On the GPU it must give the workspace entry point's results: the same kernels
run on the same plan, so outputs and caches are compared bit for bit, and
both against the fp64 oracle (max-abs 2e-2, bf16).  Two shapes run in a row,
the second smaller, so the second reads a scratch array that still holds the
first one's partials.  On the CPU: a shape beyond the scratch is refused
before anything is launched, as are the usual bad arguments.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from cached_attention_amd import flashblock as fbl
from cached_attention_amd import workloads as wl
from cached_attention_amd.session import AttentionStep

FAKE = 0x100000  # aligned fake device address: these calls fail validation first


def _raw_noalloc(desc, q=FAKE, sp=None):
    return fbl.lib().fb_step_noalloc(desc.ref, q, FAKE, FAKE, FAKE, FAKE, sp, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                     0, 1, fbl.FB_MODE_CACHED, 0, None, None)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    # eight streams of 1024-token blocks with 64 query heads on one KV head:
    # one split per stream already holds 8 * 64 * 1024 partial rows (258 MiB)
    offs = [4096 * b for b in range(9)]
    d = fbl.Desc(fbl.FB_BF16, 8, 64, 1, 128, 1024, offs, 0x10000)
    need = fbl.fb_workspace_size(d, None)
    assert need > fbl.FB_NOALLOC_SCRATCH_BYTES
    assert _raw_noalloc(d) == fbl.FB_ERR_WORKSPACE
    msg = fbl.lib().fb_last_error().decode()
    assert "fb_step_noalloc" in msg and str(need) in msg and str(fbl.FB_NOALLOC_SCRATCH_BYTES) in msg


def test_noalloc_validates_like_fb_step():
    d = fbl.Desc(fbl.FB_BF16, 1, 32, 8, 128, 64, [0, 4096], 0x10000)
    assert fbl.fb_workspace_size(d, None) <= fbl.FB_NOALLOC_SCRATCH_BYTES
    assert _raw_noalloc(d, q=None) == fbl.FB_ERR_NULL
    assert _raw_noalloc(d, q=FAKE + 8) == fbl.FB_ERR_ALIGN
    bad = fbl.Desc(fbl.FB_BF16, 1, 30, 8, 128, 64, [0, 4096], 0x10000)
    assert _raw_noalloc(bad) == fbl.FB_ERR_SHAPE


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device="cuda", dtype=dtype)


def _both_paths(w, r, chunks=None):
    """All steps of one block through fb_step (workspace) and fb_step_noalloc
    (the scratch array), each with its own caches; returns per-step outputs."""
    prefix, blocks = wl.make_inputs(w)
    blk = blocks[0]
    ch = None if chunks is None else torch.from_numpy(chunks)
    st_ws = AttentionStep(w.dtype, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets, chunks=ch)
    st_na = AttentionStep(w.dtype, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets, chunks=ch)
    t = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kp, vp = dev(prefix.k, t), dev(prefix.v, t)
    ref = oracle.run_block(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                           r=r, chunks=chunks)
    for s in range(w.steps):
        q, k, v = dev(blk.q[s], t), dev(blk.k[s], t), dev(blk.v[s], t)
        a = st_ws.step(q, k, v, kp, vp, s, r)
        b = fbl.fb_step_noalloc(st_na.desc, q, k, v, kp, vp, st_na.sparse, st_na.o_ext, st_na.lse_ext, st_na.o_res,
                                st_na.lse_res, st_na.o, st_na.lse, s, r, fbl.FB_MODE_CACHED, False)
        torch.cuda.synchronize()
        assert a == b == (s % r == 0)
        for name in ("o", "lse", "o_ext", "lse_ext") + (("o_res", "lse_res") if chunks is not None else ()):
            assert torch.equal(getattr(st_ws, name), getattr(st_na, name)), f"step {s}: {name} differs"
        err = np.abs(st_na.o.float().cpu().numpy() - ref.out[s]).max()
        assert err <= 2e-2, f"step {s}: max|O - O_oracle| = {err:.3e}"


@pytest.mark.gpu
def test_noalloc_matches_workspace_step_twice_second_smaller():
    # first call: GQA 32/8, two ragged streams, the sparse variant (both of its
    # split plans pass through the scratch); second: a smaller dense shape
    big = wl.Workload("na_big", "bf16", 2, 32, 8, 128, 64, 5000, 4, 0.5, 0.05, ragged=0.25, seed=91)
    lens = [int(x) for x in np.diff(wl.make_inputs(big)[0].offsets)]
    n_chunks = min(-(-l // 64) for l in lens)
    rng = np.random.default_rng(91)
    chunks = np.stack([np.stack([np.sort(rng.choice(n_chunks, 8, replace=False)) for _ in range(big.hkv)])
                       for _ in range(big.batch)]).astype(np.int32)
    _both_paths(big, 2, chunks)
    small = wl.Workload("na_small", "bf16", 1, 8, 2, 64, 16, 700, 3, 0.5, 0.05, seed=92)
    _both_paths(small, 2)
