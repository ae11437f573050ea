"""C ABI on the CPU: the library loads, exports what include/flashblock.h
declares, and rejects bad arguments before it touches the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from cached_attention_amd import flashblock as fbl

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "flashblock.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fb_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fbl.lib()
    declared = _declared()
    assert set(declared) == set(fbl.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert fbl.fb_abi_version() == fbl.FB_ABI_VERSION == 1
    assert fbl.fb_status_string(fbl.FB_ERR_WORKSPACE) == "workspace too small"


def _desc(**kw):
    args = dict(dtype=fbl.FB_BF16, batch=1, hq=32, hkv=8, head_dim=128, block_len=64,
                prefix_offsets_host=[0, 131072], prefix_offsets_dev=0x10000)
    args.update(kw)
    return fbl.Desc(**args)


FAKE = 0x100000  # aligned fake device address: every call below fails validation first


def _step(desc, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, sp=None, oe=FAKE, le=FAKE, orc=None, lrc=None,
             o=FAKE, lo=None, step=0, r=1, mode=fbl.FB_MODE_CACHED, force=0, ws=FAKE)
    a.update(kw)
    if "ws_bytes" not in a:
        a["ws_bytes"] = fbl.fb_workspace_size(desc) if desc is not None else 0
    d = None if desc is None else desc.ref
    sp = None if a["sp"] is None else a["sp"].ref
    return fbl.lib().fb_step(d, a["q"], a["k"], a["v"], a["kp"], a["vp"], sp, a["oe"], a["le"], a["orc"],
                             a["lrc"], a["o"], a["lo"], a["step"], a["r"], a["mode"], a["force"], None,
                             a["ws"], a["ws_bytes"], None)


def test_workspace_size_matches_split_plan():
    # 128K prefix, 8 KV heads, 256 rows per KV head -> 32 splits of 64 tiles
    d = _desc()
    splits = 32
    plan = 256   # a masked step's unit plan after the partials: 5 + 3 * 8 int32, 256-byte aligned
    expect = splits * 32 * 64 * 128 * 4 + splits * 32 * 64 * 4 + plan
    assert fbl.fb_workspace_size(d) == expect
    assert fbl.fb_workspace_size(_desc(prefix_offsets_host=[0, 0])) == 256   # empty prefix
    with pytest.raises(fbl.FlashBlockError):
        fbl.fb_workspace_size(_desc(hq=30))


@pytest.mark.parametrize("kw,status", [
    (dict(hq=30), fbl.FB_ERR_SHAPE),
    (dict(head_dim=96), fbl.FB_ERR_UNSUPPORTED),
    (dict(dtype=7), fbl.FB_ERR_UNSUPPORTED),
    (dict(block_len=0), fbl.FB_ERR_SHAPE),
    (dict(prefix_offsets_host=[5, 3]), fbl.FB_ERR_SHAPE),
    (dict(prefix_offsets_dev=None), fbl.FB_ERR_NULL),
    (dict(pre_strides=(1024, 3)), fbl.FB_ERR_ALIGN),
])
def test_step_rejects_bad_desc(kw, status):
    d = _desc(**kw)
    assert _step(d, ws_bytes=1 << 30) == status
    assert fbl.fb_last_error() != ""


def test_step_rejects_bad_args():
    d = _desc()
    assert _step(None) == fbl.FB_ERR_NULL
    assert _step(d, step=-1) == fbl.FB_ERR_ARG
    assert _step(d, r=0) == fbl.FB_ERR_ARG
    assert _step(d, mode=3) == fbl.FB_ERR_ARG
    assert _step(d, q=None) == fbl.FB_ERR_NULL
    assert _step(d, q=FAKE + 8) == fbl.FB_ERR_ALIGN
    assert _step(d, ws_bytes=fbl.fb_workspace_size(d) - 1) == fbl.FB_ERR_WORKSPACE
    assert _step(d, ws=FAKE + 64) == fbl.FB_ERR_ALIGN
    d.c.abi_version = 2
    assert _step(d, ws_bytes=1 << 30) == fbl.FB_ERR_ARG


def test_sparse_validation():
    d = _desc()
    sp = fbl.Sparse(FAKE, 205, 64)
    assert _step(d, sp=sp) == fbl.FB_ERR_NULL  # residual caches missing
    bad = fbl.Sparse(FAKE, 205, 96)
    assert _step(d, sp=bad, orc=FAKE, lrc=FAKE) == fbl.FB_ERR_ARG
    bad = fbl.Sparse(FAKE, 0, 64)
    assert _step(d, sp=bad, orc=FAKE, lrc=FAKE) == fbl.FB_ERR_ARG
    # workspace for the sparse plan is the larger of the two chunk modes
    assert fbl.fb_workspace_size(d, sp) >= 256
    prefix_bad_mode = fbl.Sparse(FAKE, 4, 64, mode=0)
    st = fbl.lib().fb_prefix_attn(d.ref, FAKE, FAKE, FAKE, prefix_bad_mode.ref, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == fbl.FB_ERR_ARG


def test_block_attn_and_merge_validation():
    d = _desc()
    lib = fbl.lib()
    assert lib.fb_block_attn(d.ref, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None) == fbl.FB_ERR_NULL
    assert lib.fb_block_attn(d.ref, FAKE, FAKE, FAKE + 4, None, None, FAKE, None, None) == fbl.FB_ERR_ALIGN
    assert lib.fb_merge(10, 98, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == fbl.FB_ERR_UNSUPPORTED
    assert lib.fb_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == fbl.FB_ERR_SHAPE
    assert lib.fb_merge(10, 128, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == fbl.FB_ERR_NULL
    assert lib.fb_merge(0, 128, None, None, None, None, None, None, None) == fbl.FB_OK


def test_prefix_combine_validation():
    """The split combine reads and writes 16-byte vectors: o_ext and the extra
    partial must be 16-byte aligned; extra_o / extra_lse come together."""
    d = _desc()
    lib = fbl.lib()
    wsb = fbl.fb_workspace_size(d)
    comb = lambda oe=FAKE, eo=None, el=None: lib.fb_prefix_combine(d.ref, None, eo, el, oe, FAKE, FAKE, wsb, None)
    assert comb(oe=FAKE + 8) == fbl.FB_ERR_ALIGN
    assert comb(eo=FAKE + 4, el=FAKE) == fbl.FB_ERR_ALIGN
    assert comb(eo=FAKE, el=None) == fbl.FB_ERR_NULL
    assert comb(oe=None) == fbl.FB_ERR_NULL


def test_desc_struct_layout():
    # fb_desc: 7 int32 + float, 2 pointers, 8 int64 strides
    assert ctypes.sizeof(fbl.fb_desc) == 32 + 16 + 64
    assert fbl.fb_desc.prefix_offsets_host.offset == 32
    assert fbl.fb_desc.q_stride_b.offset == 48
    assert ctypes.sizeof(fbl.fb_sparse) == 24


def test_adaptive_reuse_validation():
    d = _desc()
    lib = fbl.lib()
    ws_b = fbl.fb_workspace_size(d)
    tau = lambda **kw: lib.fb_refresh_mask_tau(
        kw.get("d", d.ref), FAKE, FAKE, kw.get("kc", FAKE), FAKE, kw.get("eps", 0.1), 3, kw.get("step", 1),
        kw.get("cnt", FAKE), kw.get("mask", FAKE), kw.get("ws", FAKE), kw.get("wsb", ws_b), None)
    assert tau(d=None) == fbl.FB_ERR_NULL
    assert tau(step=-1) == fbl.FB_ERR_ARG
    assert tau(eps=-1.0) == fbl.FB_ERR_ARG
    assert tau(eps=float("nan")) == fbl.FB_ERR_ARG
    assert tau(mask=None) == fbl.FB_ERR_NULL
    assert tau(kc=FAKE + 8) == fbl.FB_ERR_ALIGN   # rows move as 16-byte vectors
    assert tau(wsb=1 * 64 * 4 - 1) == fbl.FB_ERR_WORKSPACE   # B * Lb int32 flags
    assert ws_b >= 1 * 64 * 4
    gam = lambda **kw: lib.fb_refresh_mask_gamma(kw.get("d", d.ref), FAKE, kw.get("qr", FAKE),
                                                 kw.get("g", 0.9), kw.get("step", 1), FAKE, FAKE, None)
    assert gam(d=None) == fbl.FB_ERR_NULL
    assert gam(qr=None) == fbl.FB_ERR_NULL
    assert gam(g=float("nan")) == fbl.FB_ERR_ARG
    assert gam(step=-2) == fbl.FB_ERR_ARG
    sm = lambda **kw: lib.fb_step_masked(d.ref, kw.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, kw.get("mask", FAKE),
                                         FAKE, FAKE, FAKE, None, kw.get("ws", FAKE), kw.get("wsb", ws_b), None)
    assert sm(mask=None) == fbl.FB_ERR_NULL
    assert sm(q=FAKE + 2) == fbl.FB_ERR_ALIGN
    assert sm(wsb=ws_b - 1) == fbl.FB_ERR_WORKSPACE


def test_append_block_validation():
    d = _desc()
    lib = fbl.lib()
    assert lib.fb_append_block(d.ref, FAKE, FAKE, FAKE, FAKE, None, None) == fbl.FB_ERR_NULL
    assert lib.fb_append_block(d.ref, FAKE, FAKE + 8, FAKE, FAKE, FAKE, None) == fbl.FB_ERR_ALIGN
    assert lib.fb_append_block(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == fbl.FB_ERR_NULL


def test_select_chunks_validation():
    d = _desc()   # one stream of 131072 tokens: 2048 chunks of 64
    lib = fbl.lib()
    wsb = fbl.fb_select_chunks_ws(d, 64)
    assert wsb == 2048 * 8 * 128 * 4 + 2048 * 8 * 4    # pooled keys + scores, both 256-aligned here
    sel = lambda **kw: lib.fb_select_chunks(
        kw.get("d", d.ref), kw.get("q", FAKE), FAKE, kw.get("cl", 64), kw.get("k", 205), kw.get("idx", FAKE),
        kw.get("ws", FAKE), kw.get("wsb", wsb), None)
    assert sel(d=None) == fbl.FB_ERR_NULL
    assert sel(cl=0) == fbl.FB_ERR_ARG
    assert sel(k=0) == fbl.FB_ERR_ARG
    assert sel(k=2049) == fbl.FB_ERR_ARG             # more chunks asked for than the stream has
    assert sel(idx=None) == fbl.FB_ERR_NULL
    assert sel(q=FAKE + 2) == fbl.FB_ERR_ALIGN
    assert sel(wsb=wsb - 1) == fbl.FB_ERR_WORKSPACE
    assert sel(cl=4) == fbl.FB_ERR_SHAPE              # 32768 chunks: beyond the in-LDS top-k
    assert lib.fb_select_chunks_ws(d.ref, 0) == 0 and fbl.fb_last_error() != ""
    with pytest.raises(fbl.FlashBlockError):
        fbl.fb_select_chunks_ws(d, 0)


def test_pool_and_select_pooled_validation():
    d = _desc()   # 2048 chunks of 64
    lib = fbl.lib()
    pool = lambda **kw: lib.fb_pool_chunk_keys(d.ref, kw.get("kp", FAKE), kw.get("cl", 64), kw.get("cap", 2048),
                                               kw.get("first", 0), kw.get("pooled", FAKE), None)
    assert pool(cap=2047) == fbl.FB_ERR_ARG
    assert pool(first=-1) == fbl.FB_ERR_ARG
    assert pool(cl=0) == fbl.FB_ERR_ARG
    assert pool(pooled=None) == fbl.FB_ERR_NULL
    assert pool(pooled=FAKE + 4) == fbl.FB_ERR_ALIGN
    assert pool(first=2048) == fbl.FB_OK            # nothing left to pool: no launch
    sp = lambda **kw: lib.fb_select_chunks_pooled(d.ref, kw.get("q", FAKE), kw.get("pooled", FAKE), 64,
                                                  kw.get("cap", 2048), kw.get("k", 205), kw.get("sc", FAKE),
                                                  kw.get("idx", FAKE), None)
    assert sp(cap=100) == fbl.FB_ERR_ARG
    assert sp(k=0) == fbl.FB_ERR_ARG
    assert sp(k=4096) == fbl.FB_ERR_ARG
    assert sp(sc=None) == fbl.FB_ERR_NULL
    assert sp(pooled=None) == fbl.FB_ERR_NULL
    assert sp(pooled=FAKE + 8) == fbl.FB_ERR_ALIGN
    assert sp(q=FAKE + 2) == fbl.FB_ERR_ALIGN
