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
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kp = dev(prefix.k.transpose(1, 0, 2), tdt) if head_major else dev(prefix.k, tdt)
    strides = (w.head_dim, t * w.head_dim) if head_major else None
    desc = fbl.Desc(fbl.FB_BF16 if w.dtype == "bf16" else fbl.FB_F32, w.batch, w.hq, w.hkv, w.head_dim,
                    w.block_len, prefix.offsets, off_dev, pre_strides=strides)
    wsb = fbl.fb_select_chunks_ws(desc, 64)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    idx = torch.full((w.batch, w.hkv, k), -1, dtype=torch.int32, device="cuda")
    fbl.fb_select_chunks(desc, dev(q, tdt), kp, 64, k, idx, ws, wsb)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


@pytest.mark.parametrize("dtype,head_major,d", [("bf16", False, 128), ("bf16", True, 128), ("f32", False, 128),
                                               ("bf16", True, 64), ("f32", False, 64)])
def test_select_chunks_matches_oracle(dtype, head_major, d):
    w = wl.Workload("sel", dtype, 2, 8, 2, d, 16, 2000, 2, 1.0, 0.1, ragged=0.25, seed=71)
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


def _pool_gpu(w, k_dev, offsets, off_dev, cap, first, pooled, strides=None, chunk_len=64):
    desc = fbl.Desc(fbl.FB_BF16, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, offsets, off_dev,
                    pre_strides=strides)
    fbl.fb_pool_chunk_keys(desc, k_dev, chunk_len, cap, first, pooled)
    return desc


def test_pooled_keys_match_oracle():
    w = wl.Workload("pool", "bf16", 3, 8, 2, 128, 16, 700, 1, 1.0, 0.1, ragged=0.4, seed=77)
    prefix, _ = wl.make_inputs(w)
    off_dev = torch.tensor(prefix.offsets, dtype=torch.int64, device="cuda")
    n = [-(-int(prefix.offsets[b + 1] - prefix.offsets[b]) // 64) for b in range(w.batch)]
    cap = max(n) + 3
    pooled = torch.full((w.batch, cap, w.hkv, w.head_dim), 7.0, device="cuda")
    _pool_gpu(w, dev(prefix.k), prefix.offsets, off_dev, cap, 0, pooled)
    torch.cuda.synchronize()
    ref = oracle.pooled_chunk_keys(prefix.k, prefix.offsets, 64)
    got = pooled.cpu().numpy()
    for b in range(w.batch):
        # fp32 sums of <= 64 bf16 values of magnitude <= ~5: error well under 1e-5
        np.testing.assert_allclose(got[b, :n[b]], ref[b], rtol=0, atol=1e-5)
        assert (got[b, n[b]:] == 7.0).all()   # capacity rows beyond the stream's chunks untouched


def test_incremental_pooling_after_append_is_exact():
    """Pool a ragged prefix, grow every stream by a block, re-pool from the
    first chunk any stream's block touched: bit-identical to pooling the grown
    prefix from scratch (chunks below it keep the old prefix's pooled keys)."""
    w = wl.Workload("grow", "bf16", 2, 8, 2, 128, 40, 600, 1, 1.0, 0.1, ragged=0.3, seed=79)
    prefix, blocks = wl.make_inputs(w)
    lens = [int(prefix.offsets[b + 1] - prefix.offsets[b]) for b in range(w.batch)]
    new_lens = [l + w.block_len for l in lens]
    new_off = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int64)
    grown = np.concatenate([np.concatenate([prefix.k[prefix.offsets[b]:prefix.offsets[b + 1]], blocks[0].k[-1][b]])
                            for b in range(w.batch)])
    cap = max(-(-l // 64) for l in new_lens)
    pooled = torch.zeros(w.batch, cap, w.hkv, w.head_dim, device="cuda")
    fresh = torch.zeros_like(pooled)
    old_dev = torch.tensor(prefix.offsets, dtype=torch.int64, device="cuda")
    new_dev = torch.tensor(new_off, dtype=torch.int64, device="cuda")
    _pool_gpu(w, dev(prefix.k), prefix.offsets, old_dev, cap, 0, pooled)
    first = min(lens) // 64
    assert first > 0
    k_new = dev(grown)
    _pool_gpu(w, k_new, new_off, new_dev, cap, first, pooled)
    _pool_gpu(w, k_new, new_off, new_dev, cap, 0, fresh)
    torch.cuda.synchronize()
    for b in range(w.batch):
        nb = -(-new_lens[b] // 64)
        assert torch.equal(pooled[b, :nb], fresh[b, :nb]), f"stream {b}"


def test_select_pooled_equals_one_shot_and_oracle():
    w = wl.Workload("selp", "bf16", 2, 8, 2, 128, 16, 2000, 2, 1.0, 0.1, ragged=0.25, seed=71)
    prefix, blocks = wl.make_inputs(w)
    q = blocks[0].q[0]
    k = 4
    _margin_ok(q, prefix.k, prefix.offsets, k)
    off_dev = torch.tensor(prefix.offsets, dtype=torch.int64, device="cuda")
    cap = 40
    pooled = torch.zeros(w.batch, cap, w.hkv, w.head_dim, device="cuda")
    desc = _pool_gpu(w, dev(prefix.k), prefix.offsets, off_dev, cap, 0, pooled)
    scores = torch.zeros(w.batch, w.hkv, cap, device="cuda")
    idx = torch.full((w.batch, w.hkv, k), -1, dtype=torch.int32, device="cuda")
    fbl.fb_select_chunks_pooled(desc, dev(q), pooled, 64, cap, k, scores, idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), _select_gpu(w, prefix, q, k))
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.select_chunks(q, prefix.k, prefix.offsets, k, 64))
    # the scores themselves against the oracle's (fp32 accumulation of exact products)
    ref_sc = oracle.chunk_scores(q, oracle.pooled_chunk_keys(prefix.k, prefix.offsets, 64))
    sc = scores.cpu().numpy()
    for b in range(w.batch):
        n = ref_sc[b].shape[1]
        np.testing.assert_allclose(sc[b, :, :n], ref_sc[b], rtol=1e-5, atol=1e-5)


def test_select_exact_ties_go_to_lower_index():
    """Duplicate chunks score exactly alike on both sides; k is set so that the
    k-th place falls inside the tied group, which the lower indices win."""
    w = wl.Workload("ties", "bf16", 1, 4, 1, 128, 16, 64 * 40, 1, 1.0, 0.1, seed=83)
    prefix, blocks = wl.make_inputs(w)
    kp = prefix.k.copy()
    for c in (3, 11, 17, 30):   # chunks 3, 11, 17, 30 copy chunk 7
        kp[64 * c:64 * (c + 1)] = kp[64 * 7:64 * 8]
    q = blocks[0].q[0]
    sc = oracle.chunk_scores(q, oracle.pooled_chunk_keys(kp, prefix.offsets, 64))[0][0]
    better = int((sc > sc[7]).sum())
    assert (sc == sc[7]).sum() == 5
    k = better + 2   # two of the five tied chunks: 3 and 7
    p2 = wl.Prefix(kp, prefix.v, prefix.offsets)
    got = _select_gpu(w, p2, q, k)
    ref = oracle.select_chunks(q, kp, prefix.offsets, k, 64)
    np.testing.assert_array_equal(got, ref)
    assert 3 in got[0, 0] and 7 in got[0, 0] and 11 not in got[0, 0]


def test_select_at_chunk_limit():
    """16384 chunks per stream (the in-LDS limit), 1000 kept."""
    w = wl.Workload("selmax", "bf16", 1, 4, 2, 128, 16, 131072, 1, 1.0, 0.1, seed=82)
    rng = np.random.default_rng(w.seed)
    prefix = wl.make_prefix(w, rng)
    q = wl.make_block_steps(w, rng).q[0]
    k = 1000
    _margin_ok(q, prefix.k, prefix.offsets, k, chunk_len=8)
    off_dev = torch.tensor(prefix.offsets, dtype=torch.int64, device="cuda")
    desc = fbl.Desc(fbl.FB_BF16, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets, off_dev)
    wsb = fbl.fb_select_chunks_ws(desc, 8)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    idx = torch.full((1, w.hkv, k), -1, dtype=torch.int32, device="cuda")
    fbl.fb_select_chunks(desc, dev(q), dev(prefix.k), 8, k, idx, ws, wsb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.select_chunks(q, prefix.k, prefix.offsets, k, 8))
