"""The seeded input generator: bf16 rounding, determinism and structure."""
import numpy as np
import torch

from cached_attention_amd import workloads as wl


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * 3
    # exact ties: 1 + 2^-8 sits halfway between two bf16 values
    ties = (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 64, 2, dtype=np.float32))
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ours = wl.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(wl.round_bf16(np.array([np.nan], np.float32)))[0]
    bits = wl.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(back, ours)


def test_generator_is_deterministic_and_bf16_exact():
    w = wl.ci_version(wl.WORKLOADS["batched_64k"], prefix_len=300, batch=3)
    p1, b1 = wl.make_inputs(w)
    p2, b2 = wl.make_inputs(w)
    np.testing.assert_array_equal(p1.k, p2.k)
    np.testing.assert_array_equal(b1[0].q, b2[0].q)
    assert np.array_equal(wl.round_bf16(p1.v), p1.v)
    assert np.array_equal(wl.round_bf16(b1[0].k[3]), b1[0].k[3])
    lens = p1.lengths
    assert all(225 <= x <= 375 for x in lens) and len(set(lens)) > 1
    assert p1.k.shape == (sum(lens), w.hkv, w.head_dim)
    assert b1[0].q.shape == (w.steps, 3, w.block_len, w.hq, w.head_dim)


def test_random_walk_moves_by_sigma():
    w = wl.ci_version(wl.WORKLOADS["tiny_f32"], prefix_len=64)
    _, blocks = wl.make_inputs(w)
    dq = blocks[0].q[1] - blocks[0].q[0]
    assert 0.08 < dq.std() < 0.12            # sigma = 0.1, fp32 walk
    assert 0.9 < blocks[0].q[0].std() < 1.1  # N(0, 1) start


def test_chunk_selection():
    w = wl.WORKLOADS["text_gqa_128k"]
    sel = wl.make_chunk_selection(w, [131072])
    assert sel.shape == (1, 8, 205)
    for g in range(8):
        s = sel[0, g]
        assert np.all(np.diff(s) > 0) and s[0] >= 0 and s[-1] < 2048
