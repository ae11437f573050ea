"""GPU parity of the adaptive reuse policies through the C ABI against the fp64 oracle.

The masks are integer decisions: compared exactly.  Counts of updated tokens
compare exactly (|cur - prev| of bf16 / fp32 values against eps); head
similarities use fp64 sums on both sides, and each test first checks on the
oracle side that no similarity sits within 1e-4 of gamma, so both sides take
the same decision.  Outputs: bf16 max-abs 2e-2, fp32 1e-5 * max(1, max|O|).
Inputs: the decoding-style block generator (seeded); expected values: oracle only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from cached_attention_amd import flashblock as fbl
from cached_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device="cuda", dtype=dtype)


def tol(w, ref):
    return 2e-2 if w.dtype == "bf16" else 1e-5 * max(1.0, float(np.abs(ref).max()))


def _setup(dtype, batch, hq, hkv, d, lb, lp, steps, sigma, seed, head_spread=0.0, reveal=True, ragged=0.25):
    w = wl.Workload("pol", dtype, batch, hq, hkv, d, lb, lp, steps, 1.0, sigma,
                    ragged=ragged if batch > 1 else 0.0, seed=seed)
    rng = np.random.default_rng(seed)
    prefix = wl.make_prefix(w, rng)
    blk = wl.make_block_steps_decoding(w, rng, head_spread, reveal)
    return w, prefix, blk


class Gpu:
    """Device buffers of one block run."""

    def __init__(self, w, prefix, blk):
        t = TDT[w.dtype]
        self.w = w
        self.off = torch.tensor(prefix.offsets, dtype=torch.int64, device="cuda")
        self.desc = fbl.Desc(fbl.FB_BF16 if w.dtype == "bf16" else fbl.FB_F32, w.batch, w.hq, w.hkv,
                             w.head_dim, w.block_len, prefix.offsets, self.off)
        self.kp, self.vp = dev(prefix.k, t), dev(prefix.v, t)
        self.q = [dev(blk.q[s], t) for s in range(w.steps)]
        self.k = [dev(blk.k[s], t) for s in range(w.steps)]
        self.v = [dev(blk.v[s], t) for s in range(w.steps)]
        self.ws_bytes = fbl.fb_workspace_size(self.desc)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.o_ext = torch.zeros(w.batch, w.hq, w.block_len, w.head_dim, device="cuda")
        self.lse_ext = torch.full((w.batch, w.hq, w.block_len), -math.inf, device="cuda")
        self.o = torch.empty(w.batch, w.block_len, w.hq, w.head_dim, device="cuda", dtype=t)
        self.lse = torch.empty(w.batch, w.hq, w.block_len, device="cuda")
        self.mask = torch.zeros(w.batch, w.hkv, dtype=torch.int32, device="cuda")
        self.count = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
        self.sim = torch.zeros(w.batch, w.hq, device="cuda")
        self.q_ref = torch.zeros(w.batch, w.block_len, w.hq, w.head_dim, device="cuda", dtype=t)

    def tau(self, s, eps, tau):
        prev = max(s - 1, 0)
        fbl.fb_refresh_mask_tau(self.desc, self.k[prev], self.v[prev], self.k[s], self.v[s], eps, tau, s,
                                self.count, self.mask, self.ws, self.ws_bytes)

    def gamma(self, s, gamma):
        fbl.fb_refresh_mask_gamma(self.desc, self.q[s], self.q_ref, gamma, s, self.sim, self.mask)

    def step(self, s):
        fbl.fb_step_masked(self.desc, self.q[s], self.k[s], self.v[s], self.kp, self.vp, self.mask, self.o_ext,
                           self.lse_ext, self.o, self.lse, self.ws, self.ws_bytes)


@pytest.mark.parametrize("dtype,d,seed", [("bf16", 128, 41), ("f32", 128, 41), ("bf16", 64, 42)])
def test_tau_mask_counts_exact(dtype, d, seed):
    w, p, blk = _setup(dtype, 2, 8, 2, d, 40, 300, 6, 0.05, seed=seed)
    g = Gpu(w, p, blk)
    eps, tau = 0.5, 7
    ref = oracle.run_block_policy(p.k, p.v, p.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                                  "tau", tau=tau, eps=eps)
    seen = set()
    for s in range(w.steps):
        g.tau(s, eps, tau)
        torch.cuda.synchronize()
        assert g.count.cpu().numpy().tolist() == ref.counts[s].tolist(), f"step {s}"
        np.testing.assert_array_equal(g.mask.cpu().numpy(), ref.masks[s])
        seen.add(int(ref.masks[s][0, 0]))
    assert seen == {0, 1}   # the threshold both reuses and recomputes in this block


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tau_mask_counts_exact_long_block(dtype):
    """A 300-token block with head_dim 64, bf16 and fp32 (4 or 8 elements per
    16-byte vector): per-stream counts and masks compared exactly, with the
    threshold both reusing and recomputing."""
    w, p, blk = _setup(dtype, 2, 8, 2, 64, 300, 300, 6, 0.05, seed=41)
    g = Gpu(w, p, blk)
    eps, tau = 0.5, 60
    ref = oracle.run_block_policy(p.k, p.v, p.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                                  "tau", tau=tau, eps=eps)
    seen = set()
    for s in range(w.steps):
        g.tau(s, eps, tau)
        torch.cuda.synchronize()
        assert g.count.cpu().numpy().tolist() == ref.counts[s].tolist(), f"step {s}"
        np.testing.assert_array_equal(g.mask.cpu().numpy(), ref.masks[s])
        seen.add(int(ref.masks[s][0, 0]))
    assert seen == {0, 1}


def _gamma_case(dtype="bf16"):
    w, p, blk = _setup(dtype, 1, 6, 6, 128, 100, 200, 5, 0.1, seed=43, head_spread=0.9, reveal=False)
    gamma = 0.993
    ref = oracle.run_block_policy(p.k, p.v, p.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                                  "gamma", gamma=gamma)
    for s in range(1, w.steps):
        assert np.abs(ref.sims[s] - gamma).min() > 1e-4, "similarity too close to gamma for an exact compare"
    masks = np.array(ref.masks[1:])
    assert masks.min() == 0 and masks.max() == 1   # mixed: some heads reuse, some recompute
    return w, p, blk, gamma, ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gamma_mask_and_reference_queries(dtype):
    w, p, blk, gamma, ref = _gamma_case(dtype)
    g = Gpu(w, p, blk)
    q_ref = None
    for s in range(w.steps):
        g.gamma(s, gamma)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(g.mask.cpu().numpy(), ref.masks[s])
        if s > 0:
            np.testing.assert_allclose(g.sim.cpu().numpy(), ref.sims[s], rtol=0, atol=1e-6)
        # reference queries: the current ones for recomputed heads, unchanged otherwise
        if q_ref is None:
            q_ref = blk.q[0].copy()
        for h in range(w.hq):
            if ref.masks[s][0, h]:
                q_ref[0, :, h, :] = blk.q[s][0, :, h, :]
        np.testing.assert_array_equal(g.q_ref.float().cpu().numpy(), q_ref)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("f32", 64)])
def test_step_masked_tau_policy(dtype, d):
    w, p, blk = _setup(dtype, 2, 8, 2, d, 40, 300, 6, 0.05, seed=47)
    g = Gpu(w, p, blk)
    eps, tau = 0.5, 7
    ref = oracle.run_block_policy(p.k, p.v, p.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                                  "tau", tau=tau, eps=eps)
    for s in range(w.steps):
        g.tau(s, eps, tau)
        before = g.o_ext.clone()
        g.step(s)
        torch.cuda.synchronize()
        tl = tol(w, ref.out[s])
        err = np.abs(g.o.float().cpu().numpy() - ref.out[s]).max()
        assert err <= tl, f"step {s}: max|O - O_ref| = {err:.3e}"
        np.testing.assert_allclose(g.o_ext.cpu().numpy(), ref.o_ext[s], rtol=0, atol=tl)
        mask = ref.masks[s]
        for b in range(w.batch):
            for kvh in range(w.hkv):
                if not mask[b, kvh]:   # reused: the cache rows are untouched, bit for bit
                    hs = slice(kvh * (w.hq // w.hkv), (kvh + 1) * (w.hq // w.hkv))
                    assert torch.equal(g.o_ext[b, hs], before[b, hs])


def test_step_masked_gamma_policy():
    w, p, blk, gamma, ref = _gamma_case()
    g = Gpu(w, p, blk)
    for s in range(w.steps):
        g.gamma(s, gamma)
        g.step(s)
        torch.cuda.synchronize()
        err = np.abs(g.o.float().cpu().numpy() - ref.out[s]).max()
        assert err <= 2e-2, f"step {s}: max|O - O_ref| = {err:.3e}"
        lerr = np.abs(g.lse.cpu().numpy() - ref.lse[s]).max()
        assert lerr <= 2e-2, f"step {s}: LSE err {lerr:.3e}"


def test_step_masked_given_pattern_partitions_heads():
    """A fixed mask after step 0: heads of recomputed KV heads follow full
    recompute, the others keep the step-0 cache (oracle "given" policy)."""
    w, p, blk = _setup("bf16", 2, 6, 3, 128, 24, 260, 4, 0.05, seed=53)
    g = Gpu(w, p, blk)
    pattern = np.array([[1, 0, 1], [0, 1, 0]], dtype=np.int32)
    masks = [np.ones((2, 3), np.int32)] + [pattern] * (w.steps - 1)
    ref = oracle.run_block_policy(p.k, p.v, p.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                                  "given", masks=masks)
    for s in range(w.steps):
        g.mask.copy_(torch.from_numpy(masks[s]))
        g.step(s)
        torch.cuda.synchronize()
        err = np.abs(g.o.float().cpu().numpy() - ref.out[s]).max()
        assert err <= 2e-2, f"step {s}: max|O - O_ref| = {err:.3e}"


@pytest.mark.parametrize("pattern", [[[0, 0, 0], [0, 0, 0]], [[0, 0, 0], [0, 1, 0]], [[1, 1, 1], [1, 1, 1]],
                                     [[1, 0, 0], [0, 0, 1]]],
                         ids=["none", "one_pair", "all", "one_per_stream"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_masked_unit_plan(pattern, dtype):
    """Masked steps over two ragged ~3000-token prefixes (dozens of tiles per
    pair): only the listed (stream, KV head) pairs are recomputed, their
    splits spread over the whole grid; the others' cache rows stay bit for bit,
    and every output follows the oracle's given-mask run."""
    w, p, blk = _setup(dtype, 2, 6, 3, 128 if dtype == "bf16" else 64, 24, 3000, 3, 0.05, seed=57)
    g = Gpu(w, p, blk)
    pat = np.array(pattern, dtype=np.int32)
    masks = [np.ones((2, 3), np.int32)] + [pat] * (w.steps - 1)
    ref = oracle.run_block_policy(p.k, p.v, p.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                                  "given", masks=masks)
    G = w.hq // w.hkv
    for s in range(w.steps):
        before = (g.o_ext.clone(), g.lse_ext.clone())
        g.mask.copy_(torch.from_numpy(masks[s]))
        g.step(s)
        torch.cuda.synchronize()
        for b in range(w.batch):
            for kvh in range(w.hkv):
                if not masks[s][b, kvh]:
                    hs = slice(kvh * G, (kvh + 1) * G)
                    assert torch.equal(g.o_ext[b, hs], before[0][b, hs]), f"step {s}: cache of ({b}, {kvh}) moved"
                    assert torch.equal(g.lse_ext[b, hs], before[1][b, hs])
        err = np.abs(g.o.float().cpu().numpy() - ref.out[s]).max()
        assert err <= tol(w, ref.out[s]), f"step {s}: max|O - O_ref| = {err:.3e}"


def test_step_masked_many_pairs():
    """More (stream, KV head) pairs than the unit-plan workgroup has threads
    (36 streams x 8 KV heads = 288 > 256), so the plan is built over two
    chunks of pairs: a seeded mixed mask recomputes exactly its pairs, the
    others' cache rows stay bit for bit, and every output follows the oracle."""
    w, p, blk = _setup("bf16", 36, 8, 8, 64, 4, 200, 2, 0.05, seed=61)
    g = Gpu(w, p, blk)
    rng = np.random.default_rng(62)
    mixed = (rng.random((w.batch, w.hkv)) < 0.4).astype(np.int32)
    assert 0 < mixed.sum() < mixed.size and w.batch * w.hkv > 256
    masks = [np.ones((w.batch, w.hkv), np.int32), mixed]
    ref = oracle.run_block_policy(p.k, p.v, p.offsets, blk.q, blk.k, blk.v, 1 / math.sqrt(w.head_dim),
                                  "given", masks=masks)
    for s in range(w.steps):
        before = (g.o_ext.clone(), g.lse_ext.clone())
        g.mask.copy_(torch.from_numpy(masks[s]))
        g.step(s)
        torch.cuda.synchronize()
        keep = torch.from_numpy(masks[s] == 0).to("cuda")   # [B][Hkv], G = 1
        assert torch.equal(g.o_ext[keep], before[0][keep]), f"step {s}: a reused cache row moved"
        assert torch.equal(g.lse_ext[keep], before[1][keep])
        err = np.abs(g.o.float().cpu().numpy() - ref.out[s]).max()
        assert err <= tol(w, ref.out[s]), f"step {s}: max|O - O_ref| = {err:.3e}"
