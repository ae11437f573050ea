"""GPU parity of the on-device chunk selection for the sparse variant.

The selected chunk sets are integer results of floating-point scores: the GPU
scores in fp32, the oracle in fp64, so every test first checks on the oracle
side that the k-th and (k+1)-th best scores of each (stream, KV head) differ by
more than 2e-5 (relative), far above fp32 rounding of a 128-term dot product;
then the chunk lists must match exactly.  A sparse step driven by the GPU's
selection must match the oracle's sparse run on the oracle's selection.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from cached_attention_amd import flashblock as fbl
from cached_attention_amd import workloads as wl
from cached_attention_amd.session import AttentionStep

pytestmark = pytest.mark.gpu


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device="cuda", dtype=dtype)


def _margin_ok(q, k_pre, off, k, chunk_len=64):
    sc = oracle.chunk_scores(q, oracle.pooled_chunk_keys(k_pre, off, chunk_len))
    for b in range(len(sc)):
        for g in range(sc[b].shape[0]):
            s = np.sort(sc[b][g])[::-1]
            assert (s[k - 1] - s[k]) / max(1.0, abs(s[k - 1])) > 2e-5, "scores too close for an exact compare"


def _select_gpu(w, prefix, q, k, head_major=False):
    t = prefix.k.shape[0]
    off_dev = torch.tensor(prefix.offsets, dtype=torch.int64, device="cuda")
    kp = dev(prefix.k.transpose(1, 0, 2)) if head_major else dev(prefix.k)
    strides = (w.head_dim, t * w.head_dim) if head_major else None
    desc = fbl.Desc(fbl.FB_BF16, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets, off_dev,
                    pre_strides=strides)
    wsb = fbl.fb_select_chunks_ws(desc, 64)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    idx = torch.full((w.batch, w.hkv, k), -1, dtype=torch.int32, device="cuda")
    fbl.fb_select_chunks(desc, dev(q), kp, 64, k, idx, ws, wsb)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


@pytest.mark.parametrize("head_major", [False, True])
def test_select_chunks_matches_oracle(head_major):
    w = wl.Workload("sel", "bf16", 2, 8, 2, 128, 16, 2000, 2, 1.0, 0.1, ragged=0.25, seed=71)
    prefix, blocks = wl.make_inputs(w)
    q = blocks[0].q[0]
    k = 4
    _margin_ok(q, prefix.k, prefix.offsets, k)
    got = _select_gpu(w, prefix, q, k, head_major)
    ref = oracle.select_chunks(q, prefix.k, prefix.offsets, k, 64)
    np.testing.assert_array_equal(got, ref)


def test_select_then_sparse_step_matches_oracle():
    w = wl.Workload("sel2", "bf16", 2, 8, 2, 128, 16, 1500, 3, 1.0, 0.1, ragged=0.25, seed=73)
    prefix, blocks = wl.make_inputs(w)
    blk = blocks[0]
    k = 5
    _margin_ok(blk.q[0], prefix.k, prefix.offsets, k)
    sel = _select_gpu(w, prefix, blk.q[0], k)
    ref_sel = oracle.select_chunks(blk.q[0], prefix.k, prefix.offsets, k, 64)
    np.testing.assert_array_equal(sel, ref_sel)
    st = AttentionStep("bf16", w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets,
                       chunks=torch.from_numpy(sel))
    ref = oracle.run_block(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                           r=2, chunks=ref_sel)
    kp, vp = dev(prefix.k), dev(prefix.v)
    for s in range(w.steps):
        st.step(dev(blk.q[s]), dev(blk.k[s]), dev(blk.v[s]), kp, vp, s, 2)
        torch.cuda.synchronize()
        err = np.abs(st.o.float().cpu().numpy() - ref.out[s]).max()
        assert err <= 2e-2, f"step {s}: max|O - O_ref| = {err:.3e}"


def test_select_full_size_text_gqa_128k():
    """The sparse workload's shape: 2048 chunks per KV head, 10% kept."""
    w = wl.WORKLOADS["text_gqa_128k"]
    prefix, blocks = wl.make_inputs(w)
    q = blocks[0].q[0]
    k = math.ceil(w.sparse_keep * 2048)
    _margin_ok(q, prefix.k, prefix.offsets, k)
    got = _select_gpu(w, prefix, q, k, head_major=True)
    ref = oracle.select_chunks(q, prefix.k, prefix.offsets, k, 64)
    np.testing.assert_array_equal(got, ref)
