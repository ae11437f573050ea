"""The oracle's pins catch plausible mistakes in the oracle.

Each case copies ``oracle/`` and the pin suite into a temporary directory,
plants one slip in the copy's source (the repository's own oracle is never
touched) and runs the pins against the copy in a fresh interpreter.  A case
passes when the pins fail.  The slips are the ones a reader of the pages could
make while writing the oracle: a dropped term, a wrong sign, weight, index or
comparison, a swapped operand, an off-by-one in a token range.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (file under oracle/, text in the oracle, planted replacement)
MUTATIONS = {
    # partial attention and its log-normaliser
    "drop_scale": ("attention.py", "s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "drop_max_in_L": ("attention.py", "return a, mx + np.log(z)", "return a, np.log(z)"),
    "unnormalised": ("attention.py", "a = (p @ v) / z[:, None]", "a = (p @ v)"),
    "reversed_v": ("attention.py", "a = (p @ v) / z[:, None]", "a = (p @ v[::-1]) / z[:, None]"),
    # the merge equation
    "merge_sign": ("attention.py", "w_in = np.exp(l_in - m_safe)", "w_in = np.exp(m_safe - l_in)"),
    "merge_swapped_weights": ("attention.py",
                              "a = (w_out[..., None] * a_out + w_in[..., None] * a_in)",
                              "a = (w_in[..., None] * a_out + w_out[..., None] * a_in)"),
    "merge_L_drops_max": ("attention.py", "lse = m_safe + np.log(den_safe)", "lse = np.log(den_safe)"),
    # head grouping and the refresh schedule
    "gqa_modulo": ("attention.py", "return h // (hq // hkv)", "return h % hkv"),
    "refresh_phase": ("attention.py", 'return mode == "full" or step % r == 0',
                      'return mode == "full" or step % r == r - 1'),
    # the kept partials of a reuse step: the residual scored with the current
    # queries, and heads a mask does not recompute refreshed anyway
    "sparse_residual_current_queries": ("attention.py", "ext_o, ext_l = merge(cache_o, cache_l, sel_o, sel_l)",
                                        "ext_o, ext_l = merge(*prefix_partial(q, k_pre, v_pre, offsets, scale, "
                                        'chunks, chunk_len, "complement"), sel_o, sel_l)'),
    "policy_refreshes_unmasked": ("policies.py", "if mask[b, kv_group(h, hq, hkv)]:\n                        cache_o",
                                  "if True:\n                        cache_o"),
    # sparse token sets
    "complement_loses_token": ("attention.py", "return np.nonzero(~sel)[0]",
                               "return np.nonzero(~sel)[0][:-1]"),
    "chunk_end_off_by_one": ("attention.py", "sel[c * chunk_len: min((c + 1) * chunk_len, lp)] = True",
                             "sel[c * chunk_len: min((c + 1) * chunk_len - 1, lp)] = True"),
    # sparse attention without the cached residual (the merge itself is
    # symmetric in its two partials, so an operand swap there is no mistake)
    "sparse_only_complement": ("attention.py",
                               'prefix_partial(q_blk, k_pre, v_pre, offsets, scale, chunks, chunk_len, "selected")',
                               'prefix_partial(q_blk, k_pre, v_pre, offsets, scale, chunks, chunk_len, "complement")'),
    "sparse_only_drops_block": ("attention.py", "o, _ = merge(sel_o, sel_l, in_o, in_l)", "o = sel_o"),
    "sparse_only_drops_selected": ("attention.py", "o, _ = merge(sel_o, sel_l, in_o, in_l)", "o = in_o"),
    # growing the prefix with a finalised block
    "grow_v_from_k": ("attention.py", "vs.append(v_last[b])", "vs.append(k_last[b])"),
    "append_v_from_k": ("attention.py", "v_new[r0:r0 + lb] = v_last[b]", "v_new[r0:r0 + lb] = k_last[b]"),
    # adaptive reuse
    "updated_ignores_v": ("policies.py", "changed = (dk > eps) | (dv > eps)", "changed = (dk > eps)"),
    "tau_strict": ("policies.py", "m_count[b] >= tau", "m_count[b] > tau"),
    "gamma_inverted": ("policies.py", "not (sim[b, h] > gamma)", "sim[b, h] > gamma"),
    "cosine_wrong_norm": ("policies.py", "np.sqrt(nx * ny)", "np.sqrt(nx) * ny"),
    "gamma_reference_frozen": ("policies.py", "q_ref[b, :, h, :] = q[b, :, h, :]", "pass"),
    "gamma_reference_every_step": ("policies.py", "if mask[b, kv_group(h, hq, hkv)]:\n                        q_ref",
                                   "if True:\n                        q_ref"),
    # chunk selection
    "pooled_sum": ("policies.py", ".mean(axis=0)", ".sum(axis=0)"),
    "score_mean_over_queries": ("policies.py", "(qs @ pooled[b][:, g, :].T).max(axis=0)",
                                "(qs @ pooled[b][:, g, :].T).mean(axis=0)"),
    "ties_to_higher_index": ("policies.py", "key=lambda c: (-s[c], c)", "key=lambda c: (-s[c], -c)"),
}


def _plant(tmp_path, fname, old, new):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    tdir = tmp_path / "tests"
    tdir.mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tdir / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tdir / "golden")
    path = tmp_path / "oracle" / fname
    src = path.read_text()
    assert src.count(old) == 1, f"planting site not unique in oracle/{fname}: {old!r}"
    path.write_text(src.replace(old, new))


def _run_pins(tmp_path):
    # the copy's oracle comes first on the path; the package (seeded inputs) from the repository
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]),
               PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "tests/test_oracle_pins.py"],
                          cwd=tmp_path, env=env, capture_output=True, text=True, timeout=300)


def test_unmodified_copy_passes(tmp_path):
    """The harness itself: the copied pins pass on an untouched copy of the oracle."""
    _plant(tmp_path, "attention.py", "def merge(", "def merge(")
    r = _run_pins(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(tmp_path, name):
    fname, old, new = MUTATIONS[name]
    _plant(tmp_path, fname, old, new)
    r = _run_pins(tmp_path)
    # returncode 1: some pin failed (collection errors, 2, would not show the pins at work)
    assert r.returncode == 1, (f"pins did not catch '{name}' (exit {r.returncode}):\n"
                               + r.stdout[-2000:] + r.stderr[-2000:])
