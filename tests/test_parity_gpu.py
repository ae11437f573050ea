"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: bf16 workloads max-abs 2e-2 on O, O_ext and LSE (bf16 inputs,
fp32 accumulation); fp32 max-abs 1e-5 * max(1, max|X_oracle|) for X = O and LSE
(relative to the quantity's magnitude).  Drift parity:
|drift_gpu - drift_oracle| <= 2 * tol.  Every input comes from the seeded
generator; every expected value from the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import to_output_layout
from cached_attention_amd import flashblock as fbl
from cached_attention_amd import workloads as wl
from cached_attention_amd.session import AttentionStep

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device="cuda", dtype=dtype)


def tol(w, ref, lse=None):
    """Output bound: bf16 2e-2 absolute; fp32 1e-5 relative to max|O|.

    For fp32 the relative bound widens where the log-normalisers are large.
    The partials travel through the split combine and the cache merge as fp32
    LSEs, and each rounding of an LSE of magnitude |L| is off by up to
    |L|*2^-24 absolute.  That is a relative error of the same size in the
    partial's merge weight.  Eight such roundings bound the chain (log2 to
    natural log, the max shift, combine, merge), so the fp32 bound is
    max(1e-5, 8 * 2^-24 * max|L|) relative.  For ordinary inputs, |L| <= 20,
    this stays 1e-5.  It grows only for scores in the hundreds, as in the
    score-jump case.
    """
    if w.dtype == "bf16":
        return 2e-2
    rel = 1e-5
    if lse is not None:
        finite = np.asarray(lse)[np.isfinite(lse)]
        if finite.size:
            rel = max(rel, 8 * 2.0 ** -24 * float(np.abs(finite).max()))
    return rel * max(1.0, float(np.abs(ref).max()))


def tol_lse(w, ref_lse):
    """LSE bound: as tol(), relative to the largest finite |LSE| for fp32."""
    finite = np.isfinite(ref_lse)
    return tol(w, ref_lse[finite] if finite.any() else np.zeros(1))


def scale_of(w):
    return 1.0 / math.sqrt(w.head_dim)


class GpuResult:
    def __init__(self):
        self.out, self.lse, self.o_ext, self.lse_ext, self.refreshed = [], [], [], [], []


def run_gpu(w, prefix, blk, r=1, mode="cached", chunks=None, st=None, k_pre=None, v_pre=None):
    t = TDT[w.dtype]
    if st is None:
        st = AttentionStep(w.dtype, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets,
                           chunks=None if chunks is None else torch.from_numpy(chunks))
    kp = dev(prefix.k, t) if k_pre is None else k_pre
    vp = dev(prefix.v, t) if v_pre is None else v_pre
    res = GpuResult()
    for s in range(blk.q.shape[0]):
        q, k, v = dev(blk.q[s], t), dev(blk.k[s], t), dev(blk.v[s], t)
        res.refreshed.append(st.step(q, k, v, kp, vp, s, r, mode))
        torch.cuda.synchronize()
        res.out.append(st.o.float().cpu().numpy().astype(np.float64))
        res.lse.append(st.lse.cpu().numpy().astype(np.float64))
        res.o_ext.append(st.o_ext.cpu().numpy().astype(np.float64))
        res.lse_ext.append(st.lse_ext.cpu().numpy().astype(np.float64))
    return res


def check_block(w, prefix, blk, r, mode, chunks=None, check_cache=True):
    scale = scale_of(w)
    ref = oracle.run_block(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, scale, r=r,
                           mode=mode, chunks=chunks)
    got = run_gpu(w, prefix, blk, r, mode, chunks)
    for s in range(w.steps):
        tl = tol(w, ref.out[s], ref.lse[s])
        err = np.abs(got.out[s] - ref.out[s]).max()
        assert err <= tl, f"step {s}: max|O - O_ref| = {err:.3e} > {tl:.1e}"
        lerr = np.abs(got.lse[s] - ref.lse[s]).max()
        assert lerr <= tol_lse(w, ref.lse[s]), f"step {s}: LSE err {lerr:.3e}"
        assert got.refreshed[s] == ref.refreshed[s]
        if check_cache and mode == "cached":
            e1 = np.abs(got.o_ext[s] - ref.o_ext[s]).max()
            finite = np.isfinite(ref.lse_ext[s])
            assert np.array_equal(np.isfinite(got.lse_ext[s]), finite)
            e2 = np.abs(got.lse_ext[s][finite] - ref.lse_ext[s][finite]).max() if finite.any() else 0.0
            assert e1 <= tl and e2 <= tol_lse(w, ref.lse_ext[s]), f"step {s}: cache err {e1:.3e} {e2:.3e}"
    return ref, got


# ---------------------------------------------------------------------------
# every workload at CI sizes, exact and cached modes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("r,mode", [(1, "cached"), (2, "cached"), (4, "cached"), (1, "full")])
def test_tiny_f32(r, mode):
    w = wl.WORKLOADS["tiny_f32"]
    prefix, blocks = wl.make_inputs(w)
    check_block(w, prefix, blocks[0], r, mode)


@pytest.mark.parametrize("lp", [1000, 4096])
@pytest.mark.parametrize("r,mode", [(1, "cached"), (4, "cached"), (8, "cached"), (1, "full")])
def test_text_mha(lp, r, mode):
    w = wl.ci_version(wl.WORKLOADS["text_mha_4k"], prefix_len=lp)
    prefix, blocks = wl.make_inputs(w)
    check_block(w, prefix, blocks[0], r, mode)


@pytest.mark.parametrize("r,mode", [(1, "cached"), (8, "cached"), (1, "full")])
def test_text_gqa(r, mode):
    w = wl.ci_version(wl.WORKLOADS["text_gqa_128k"], prefix_len=4100)
    prefix, blocks = wl.make_inputs(w)
    check_block(w, prefix, blocks[0], r, mode)


@pytest.mark.parametrize("r", [1, 8])
def test_text_gqa_sparse(r):
    w = wl.ci_version(wl.WORKLOADS["text_gqa_128k"], prefix_len=4100)   # 65 chunks, last one 4 tokens
    prefix, blocks = wl.make_inputs(w)
    chunks = wl.make_chunk_selection(w, prefix.lengths)
    assert chunks.shape[-1] == 7
    chunks[0, 0, -1] = 64          # include the ragged last chunk once
    chunks[0, 0] = np.sort(chunks[0, 0])
    if len(set(chunks[0, 0].tolist())) < 7:
        chunks[0, 0] = np.array([1, 5, 9, 20, 33, 50, 64], dtype=np.int32)
    check_block(w, prefix, blocks[0], r, "cached", chunks=chunks)


@pytest.mark.parametrize("batch,hq,hkv,lb,mode", [(2, 2, 2, 1100, "cached"), (2, 8, 2, 300, "cached"),
                                                  (2, 8, 2, 300, "full"), (1, 16, 16, 1190, "cached"),
                                                  (1, 16, 16, 1025, "cached"), (1, 64, 16, 300, "cached"),
                                                  (2, 8, 8, 1190, "full"), (1, 32, 32, 1100, "cached"),
                                                  (1, 8, 8, 600, "cached")])
def test_big_block_ragged_streams(batch, hq, hkv, lb, mode):
    """Blocks of >= 1024 query rows per KV head (the key-group block
    configurations), MHA and GQA, over ragged streams, cached and full.  The
    next five need fewer rounds of 80-row workgroups than of 64-row ones,
    so they run the 80-row form: ragged in rows and keys (1190), a last key
    tile of one key, which the second key group sees fully masked (1025),
    80-row tiles that straddle query heads (GQA 64/16, 300 tokens), two
    ragged streams in full mode, and 448 workgroups of 80 rows, two rounds
    (32 x 1100).  The last has 600 rows but 600 keys: 64-row key groups."""
    w = wl.Workload("big", "bf16", batch, hq, hkv, 128, lb, 300, 3, 1.0, 0.1, ragged=0.25, seed=97)
    prefix, blocks = wl.make_inputs(w)
    check_block(w, prefix, blocks[0], 2, mode)


@pytest.mark.parametrize("r", [1, 2])
@pytest.mark.parametrize("chunk_len,d,lb", [(128, 128, 16), (64, 64, 48)], ids=["c128_d128", "c64_d64_192rows"])
def test_sparse_chunk128_ragged_batch(r, chunk_len, d, lb):
    """128-token chunks (two 64-key tiles each), and 64-token chunks at
    head_dim 64 with 192 query rows per KV head (one 256-row prefix tile),
    over two ragged streams whose last chunks are partial; GQA 8/2."""
    w = wl.Workload("sp128", "bf16", 2, 8, 2, d, lb, 1500, 3, 0.5, 0.05, ragged=0.3, seed=91,
                    sparse_keep=0.25, chunk_len=chunk_len)
    prefix, blocks = wl.make_inputs(w)
    chunks = wl.make_chunk_selection(w, prefix.lengths)
    assert chunks.shape[-1] >= 2 and all(l % chunk_len for l in prefix.lengths)
    for b in range(w.batch):   # include each stream's partial last chunk
        last = (prefix.lengths[b] - 1) // chunk_len
        for g in range(w.hkv):
            if last not in chunks[b, g]:
                chunks[b, g, -1] = last
                chunks[b, g] = np.sort(chunks[b, g])
    scale = scale_of(w)
    ref = oracle.run_block(prefix.k, prefix.v, prefix.offsets, blocks[0].q, blocks[0].k, blocks[0].v, scale, r=r,
                           chunks=chunks, chunk_len=chunk_len)
    st = AttentionStep(w.dtype, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets,
                       chunks=torch.from_numpy(chunks), chunk_len=chunk_len)
    got = run_gpu(w, prefix, blocks[0], r, "cached", st=st)
    for s in range(w.steps):
        err = np.abs(got.out[s] - ref.out[s]).max()
        assert err <= 2e-2, f"step {s}: max|O - O_ref| = {err:.3e}"
        assert np.abs(got.lse[s] - ref.lse[s]).max() <= 2e-2


@pytest.mark.parametrize("r,mode", [(1, "cached"), (4, "cached"), (1, "full")])
def test_video_frame_block(r, mode):
    w = wl.ci_version(wl.WORKLOADS["video_1560"], prefix_len=3120, hq=4, hkv=4, n_blocks=1)
    prefix, blocks = wl.make_inputs(w)
    check_block(w, prefix, blocks[0], r, mode)


def test_video_growing_prefix():
    """Two blocks; the finalised block's last-step K/V joins the prefix."""
    w = wl.ci_version(wl.WORKLOADS["video_1560"], prefix_len=1560, hq=2, hkv=2, n_blocks=2)
    prefix, blocks = wl.make_inputs(w)
    kp, vp, off = prefix.k, prefix.v, prefix.offsets
    for bi, blk in enumerate(blocks):
        p = wl.Prefix(kp, vp, off)
        check_block(w, p, blk, 4, "cached")
        kp, vp, off = oracle.grow_prefix(kp, vp, off, blk.k[-1], blk.v[-1])
    assert off[-1] == 1560 * 3


@pytest.mark.parametrize("r,mode", [(1, "cached"), (2, "cached"), (8, "cached"), (1, "full")])
def test_batched_ragged(r, mode):
    w = wl.ci_version(wl.WORKLOADS["batched_64k"], prefix_len=1000)
    prefix, blocks = wl.make_inputs(w)
    assert len(set(prefix.lengths)) > 1
    check_block(w, prefix, blocks[0], r, mode)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _custom(dtype, batch, hq, hkv, d, lb, lens, steps=2, seed=99):
    w = wl.Workload("edge", dtype, batch, hq, hkv, d, lb, 0, steps, 1.0, 0.1, seed=seed)
    rng = np.random.default_rng(seed)
    off = np.zeros(batch + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    t = int(off[-1])
    draw = (lambda s: wl.round_bf16(rng.standard_normal(s, dtype=np.float32))) if dtype == "bf16" else \
        (lambda s: rng.standard_normal(s, dtype=np.float32))
    prefix = wl.Prefix(draw((t, hkv, d)), draw((t, hkv, d)), off)
    blk = wl.make_block_steps(w, rng)
    return w, prefix, blk


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", [
    dict(batch=2, hq=4, hkv=2, d=128, lb=8, lens=[0, 0]),          # empty prefix everywhere
    dict(batch=3, hq=4, hkv=2, d=128, lb=8, lens=[10, 0, 70]),     # < 1 tile, empty, ragged
    dict(batch=1, hq=1, hkv=1, d=128, lb=1, lens=[129]),           # single query row
    dict(batch=1, hq=8, hkv=2, d=64, lb=17, lens=[300]),           # D=64, G=4, 68 rows per KV head
    dict(batch=1, hq=2, hkv=1, d=128, lb=100, lens=[64 * 5]),      # 200 rows: several row tiles
    dict(batch=2, hq=2, hkv=2, d=128, lb=300, lens=[700, 130]),    # 300 rows: three 128-row prefix tiles
    dict(batch=1, hq=4, hkv=1, d=64, lb=75, lens=[1000]),          # 300 rows at D=64
    dict(batch=2, hq=8, hkv=2, d=64, lb=48, lens=[900, 70]),       # 192 rows at D=64: one 256-row prefix tile
    dict(batch=1, hq=2, hkv=2, d=64, lb=1100, lens=[300]),         # 1100 rows at D=64: 64-row key-group block pass
    dict(batch=1, hq=16, hkv=16, d=64, lb=1190, lens=[200]),       # 16 x 1190 rows at D=64: 80-row key-group block pass
    dict(batch=1, hq=32, hkv=8, d=128, lb=8, lens=[6400]),         # 25 splits of 4 tiles: the 32-split combine
    dict(batch=2, hq=2, hkv=2, d=128, lb=1100, lens=[0, 90]),      # 64-row key groups, one stream without prefix
    dict(batch=2, hq=16, hkv=16, d=128, lb=1190, lens=[150, 0]),   # 80-row key groups, one stream without prefix
])
def test_edge_shapes(dtype, case):
    w, prefix, blk = _custom(dtype, **case)
    for r, mode in ((1, "cached"), (2, "cached"), (1, "full")):
        check_block(w, prefix, blk, r, mode)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [
    dict(hq=2, hkv=1, lb=100),   # 200 rows per KV head: the 8-wave 256-row split-KV pass; 2-tile block
    dict(hq=2, hkv=1, lb=64),    # 128 rows: two 4-wave 128-row workgroups per CU
    dict(hq=1, hkv=1, lb=32),    # 32 rows: the pipelined 16-row split-KV pass
    dict(hq=1, hkv=1, lb=1100),  # 1100 rows: the block pass's two key groups, a spike in each one's half
    dict(hq=16, hkv=16, lb=1190),  # 16 x 1190 rows: the 80-row key-group block workgroups
], ids=["rows200", "rows128", "rows32", "rows1100", "heads16_rows1190"])
def test_score_jump_reruns_pass(dtype, shape):
    """Scores far above a pass's first-tile maxima (the kernel's softmax reference).

    Prefix: 6 tiles in two splits (splits of at least 4 tiles): tiles 0-3
    and 4-5, or, in the 256-row layout, which interleaves its splits, tiles
    0, 2, 4 and 1, 3, 5; a large key in tile 3 and one in tile 5 give some
    rows scores more than 64 log2 units above their split's first-tile
    maxima (any ordinary tile's maxima are far below the spike), which sends
    the bf16 pass through its rerun against the split's exact maxima, from
    each split-KV layout's own main loop.  Block (when it has a second tile): the
    same in its second tile (key 80), and for blocks of 1024 rows and more,
    whose waves split every tile into two 32-key halves, also in the second
    half of its third tile (key 168).  Results must still match the oracle.
    """
    lb = shape["lb"]
    w, prefix, blk = _custom(dtype, batch=1, hq=shape["hq"], hkv=shape["hkv"], d=128, lb=lb, lens=[64 * 6])
    prefix.k[200] = 80.0
    prefix.k[330] = 80.0
    spikes = [t for t in (80, 168) if t < lb and (t == 80 or lb >= 1024)]
    for t in spikes:
        blk.k[:, :, t] = 80.0
    # precondition: some row's spike score clears its first tile's max by > 64 (log2)
    scale, log2e = scale_of(w), 1.0 / math.log(2.0)
    q = blk.q.astype(np.float64).reshape(-1, w.head_dim)
    for spike_tok, first_tile in ((200, 0), (330, 4), (200, 1), (330, 1)):   # first tiles of both layouts' splits
        first = (q @ prefix.k[64 * first_tile:64 * first_tile + 64, 0].astype(np.float64).T).max(axis=1)
        spike = q @ prefix.k[spike_tok, 0].astype(np.float64)
        assert ((spike - first) * scale * log2e > 64).any()
    for t in spikes:
        bfirst = np.einsum("sbthd,sbkd->sbthk", blk.q.astype(np.float64),
                           blk.k[:, :, 0:64, 0].astype(np.float64)).max(-1)
        bspike = np.einsum("sbthd,sbd->sbth", blk.q.astype(np.float64), blk.k[:, :, t, 0].astype(np.float64))
        assert ((bspike - bfirst) * scale * log2e > 64).any()
    for r, mode in ((1, "cached"), (2, "cached"), (1, "full")):
        check_block(w, prefix, blk, r, mode)


def test_r1_equals_full_bitwise_and_deterministic():
    w = wl.ci_version(wl.WORKLOADS["text_gqa_128k"], prefix_len=2000)
    prefix, blocks = wl.make_inputs(w)
    a = run_gpu(w, prefix, blocks[0], 1, "cached")
    b = run_gpu(w, prefix, blocks[0], 1, "full")
    c = run_gpu(w, prefix, blocks[0], 1, "cached")
    for s in range(w.steps):
        np.testing.assert_array_equal(a.out[s], b.out[s])
        np.testing.assert_array_equal(a.out[s], c.out[s])
        np.testing.assert_array_equal(a.lse[s], c.lse[s])


def test_drift_parity():
    w = wl.ci_version(wl.WORKLOADS["text_mha_4k"], prefix_len=2048)
    prefix, blocks = wl.make_inputs(w)
    blk = blocks[0]
    scale = scale_of(w)
    ref_c = oracle.run_block(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, scale, r=8)
    ref_f = oracle.run_block(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, scale, mode="full")
    got_c = run_gpu(w, prefix, blk, 8, "cached")
    got_f = run_gpu(w, prefix, blk, 1, "full")
    for s in range(w.steps):
        d_ref = np.abs(ref_c.out[s] - ref_f.out[s]).max()
        d_gpu = np.abs(got_c.out[s] - got_f.out[s]).max()
        assert abs(d_gpu - d_ref) <= 2 * 2e-2
        if s == 0:
            assert d_gpu == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partials_then_combine_with_extra_partial(dtype):
    """fb_prefix_partials + fb_prefix_combine called on their own, the combine
    folding in one more partial: equals the oracle's prefix partial merged with
    that partial by the merge equation (and, without it, fb_prefix_attn)."""
    w = wl.Workload("pc", dtype, 2, 8, 2, 128, 16, 700, 1, 1.0, 0.1, ragged=0.3, seed=101)
    prefix, blocks = wl.make_inputs(w)
    q = blocks[0].q[0]
    t = TDT[dtype]
    off_dev = torch.tensor(prefix.offsets, dtype=torch.int64, device="cuda")
    desc = fbl.Desc(fbl.FB_BF16 if dtype == "bf16" else fbl.FB_F32, w.batch, w.hq, w.hkv, w.head_dim, w.block_len,
                    prefix.offsets, off_dev)
    wsb = fbl.fb_workspace_size(desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(5)
    xo = rng.standard_normal((w.batch, w.hq, w.block_len, w.head_dim))
    xl = rng.standard_normal((w.batch, w.hq, w.block_len)) * 3
    xl[0, 0, :3] = -np.inf          # a few rows with an empty extra partial
    xo[0, 0, :3] = 0.0
    fx = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    oe = torch.empty(w.batch, w.hq, w.block_len, w.head_dim, device="cuda")
    le = torch.empty(w.batch, w.hq, w.block_len, device="cuda")
    fbl.fb_prefix_partials(desc, dev(q, t), dev(prefix.k, t), dev(prefix.v, t), None, ws, wsb)
    fbl.fb_prefix_combine(desc, None, fx(xo), fx(xl), oe, le, ws, wsb)
    torch.cuda.synchronize()
    po, pl = oracle.prefix_partial(q, prefix.k, prefix.v, prefix.offsets, scale_of(w))
    ro, rl = oracle.merge(po, pl, xo.astype(np.float32).astype(np.float64), xl.astype(np.float32).astype(np.float64))
    tl = 2e-2 if dtype == "bf16" else 1e-5 * max(1.0, float(np.abs(ro).max()))
    assert np.abs(oe.cpu().numpy() - ro).max() <= tl
    assert np.abs(le.cpu().numpy() - rl).max() <= (2e-2 if dtype == "bf16" else 1e-5 * max(1.0, np.abs(rl).max()))
    # without the extra partial the combine equals fb_prefix_attn
    fbl.fb_prefix_combine(desc, None, None, None, oe, le, ws, wsb)
    o2 = torch.empty_like(oe)
    l2 = torch.empty_like(le)
    fbl.fb_prefix_attn(desc, dev(q, t), dev(prefix.k, t), dev(prefix.v, t), None, o2, l2, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(oe, o2) and torch.equal(le, l2)


def test_fb_merge_matches_oracle():
    rng = np.random.default_rng(5)
    rows, d = 1000, 128
    oa, ob = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    la, lb = rng.standard_normal(rows) * 3, rng.standard_normal(rows) * 3
    la[:10] = -np.inf
    lb[5:15] = -np.inf
    oa[:10] = 0
    ob[5:15] = 0
    ref_o, ref_l = oracle.merge(oa, la, ob, lb)
    t = [torch.tensor(x, dtype=torch.float32, device="cuda") for x in (oa, la, ob, lb)]
    o = torch.empty_like(t[0])
    l = torch.empty_like(t[1])
    fbl.fb_merge(rows, d, t[0], t[1], t[2], t[3], o, l)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o.cpu().numpy(), ref_o, rtol=0, atol=1e-5)
    got_l = l.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=0, atol=1e-5)
    # in place: o aliases o_a, lse aliases lse_a
    fbl.fb_merge(rows, d, t[0], t[1], t[2], t[3], t[0], t[1])
    torch.cuda.synchronize()
    np.testing.assert_allclose(t[0].cpu().numpy(), ref_o, rtol=0, atol=1e-5)


# ---------------------------------------------------------------------------
# full-size workloads: the GPU runs everything, the oracle checks sampled heads
# ---------------------------------------------------------------------------

def _sampled_check(w, prefix, blk, heads, steps=(0,), r=1):
    """Runs the whole workload on the GPU; the oracle recomputes the listed
    (stream, query head) pairs one by one as single-head problems."""
    scale = scale_of(w)
    n = max(steps) + 1
    sub = wl.BlockSteps(blk.q[:n], blk.k[:n], blk.v[:n])
    got = run_gpu(w, prefix, sub, r, "cached")
    for (b, h) in heads:
        g = h // (w.hq // w.hkv)
        t0, t1 = int(prefix.offsets[b]), int(prefix.offsets[b + 1])
        ref = oracle.run_block(prefix.k[t0:t1, g:g + 1, :], prefix.v[t0:t1, g:g + 1, :],
                               np.array([0, t1 - t0]), sub.q[:, b:b + 1, :, h:h + 1, :],
                               sub.k[:, b:b + 1, :, g:g + 1, :], sub.v[:, b:b + 1, :, g:g + 1, :],
                               scale, r=r)
        for s in steps:
            err = np.abs(got.out[s][b, :, h, :] - ref.out[s][0, :, 0, :]).max()
            assert err <= 2e-2, f"stream {b} head {h} step {s}: {err:.3e}"
            lerr = np.abs(got.lse[s][b, h] - ref.lse[s][0, 0]).max()
            assert lerr <= 2e-2, f"stream {b} head {h} step {s}: LSE {lerr:.3e}"


@pytest.mark.slow
def test_full_size_text_gqa_128k():
    w = wl.WORKLOADS["text_gqa_128k"]
    prefix, blocks = wl.make_inputs(w)
    _sampled_check(w, prefix, blocks[0], heads=[(0, 0), (0, 13), (0, 31)])


@pytest.mark.slow
def test_full_size_batched_64k():
    w = wl.WORKLOADS["batched_64k"]
    prefix, blocks = wl.make_inputs(w)
    _sampled_check(w, prefix, blocks[0], heads=[(0, 0), (3, 17), (7, 31)])


@pytest.mark.slow
def test_full_size_text_mha_32k():
    w = wl.WORKLOADS["text_mha_32k"]
    prefix, blocks = wl.make_inputs(w)
    _sampled_check(w, prefix, blocks[0], heads=[(0, 0), (0, 31)], steps=(0, 3), r=8)


@pytest.mark.slow
def test_full_size_video():
    w = wl.WORKLOADS["video_1560"]
    prefix, blocks = wl.make_inputs(wl.ci_version(w, prefix_len=w.prefix_len, n_blocks=1))
    _sampled_check(w, prefix, blocks[0], heads=[(0, 0), (0, 11)])


@pytest.mark.parametrize("layout,dtype,d", [("token", "bf16", 128), ("head", "bf16", 128), ("token", "f32", 64),
                                            ("head", "f32", 128)])
def test_append_block_grows_prefix_exactly(layout, dtype, d):
    """The finalised block's K/V land in the grown prefix bit for bit (oracle
    grow_prefix), and the next block's step over that prefix matches the oracle."""
    w = wl.Workload("grow", dtype, 2, 8, 2, d, 24, 200, 3, 1.0, 0.1, ragged=0.25, seed=61)
    rng = np.random.default_rng(61)
    prefix = wl.make_prefix(w, rng)
    blk0, blk1 = wl.make_block_steps(w, rng), wl.make_block_steps(w, rng)
    k_last, v_last = blk0.k[-1], blk0.v[-1]
    k2, v2, off2 = oracle.grow_prefix(prefix.k, prefix.v, prefix.offsets, k_last, v_last)
    t2 = int(off2[-1])
    lens = [int(prefix.offsets[b + 1] - prefix.offsets[b]) for b in range(w.batch)]
    bf = TDT[dtype]
    # the grown buffer: old rows moved to the new layout on the device, then the append
    kd = torch.zeros(t2, w.hkv, w.head_dim, dtype=bf, device="cuda")
    vd = torch.zeros_like(kd)
    kp_old, vp_old = dev(prefix.k, bf), dev(prefix.v, bf)
    for b in range(w.batch):
        o0, o1 = int(prefix.offsets[b]), int(prefix.offsets[b + 1])
        kd[int(off2[b]):int(off2[b]) + lens[b]] = kp_old[o0:o1]
        vd[int(off2[b]):int(off2[b]) + lens[b]] = vp_old[o0:o1]
    if layout == "head":   # [Hkv][T][D]
        kd = kd.permute(1, 0, 2).contiguous()
        vd = vd.permute(1, 0, 2).contiguous()
        pre_strides = (w.head_dim, t2 * w.head_dim)
    else:
        pre_strides = None
    off_dev = torch.tensor(off2, dtype=torch.int64, device="cuda")
    desc = fbl.Desc(fbl.FB_BF16 if dtype == "bf16" else fbl.FB_F32, w.batch, w.hq, w.hkv, w.head_dim, w.block_len,
                    off2, off_dev, pre_strides=pre_strides)
    dst = torch.tensor([int(off2[b]) + lens[b] for b in range(w.batch)], dtype=torch.int64, device="cuda")
    fbl.fb_append_block(desc, dev(k_last, bf), dev(v_last, bf), kd, vd, dst)
    torch.cuda.synchronize()
    kg, vg = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    if layout == "head":
        kg, vg = kg.transpose(1, 0, 2), vg.transpose(1, 0, 2)
    np.testing.assert_array_equal(kg, k2)
    np.testing.assert_array_equal(vg, v2)
    # the next block over the grown prefix
    grown = wl.Prefix(k2, v2, off2)
    st = AttentionStep(dtype, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, off2, pre_strides=pre_strides)
    ref = oracle.run_block(k2, v2, off2, blk1.q, blk1.k, blk1.v, scale_of(w), r=2)
    got = run_gpu(w, grown, blk1, r=2, st=st, k_pre=kd, v_pre=vd)
    for s in range(w.steps):
        assert np.abs(got.out[s] - ref.out[s]).max() <= tol(w, ref.out[s])
