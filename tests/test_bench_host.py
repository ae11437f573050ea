"""bench.py host logic on the CPU: the algorithmic bytes and FLOPs that the
roofline divides by the measured time, the HBM-traffic table lookup and its
kernel-source check, and the one-GPU guard."""
import hashlib
import importlib.util
import os
import shutil
import subprocess
import sys

from cached_attention_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_bench(path):
    spec = importlib.util.spec_from_file_location("bench_under_test", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


bench = _load_bench(os.path.join(ROOT, "bench.py"))


def test_prefix_bytes_and_flops_by_hand():
    # 128K GQA: K+V 2*131072*8*128*2, Q 64*32*128*2, O_ext + LSE 32*64*(128+1)*4
    pb, pf, _, _ = bench.algorithmic(wl.WORKLOADS["text_gqa_128k"], [131072])
    assert pb == 536_870_912 + 524_288 + 1_056_768 == 538_451_968
    assert pf == 4 * 32 * 64 * 128 * 131072                      # 137.4 GFLOP
    # 32K MHA
    pb, pf, _, _ = bench.algorithmic(wl.WORKLOADS["text_mha_32k"], [32768])
    assert pb == 2 * 32768 * 32 * 128 * 2 + 32 * 32 * 128 * 2 + 32 * 32 * 129 * 4 == 537_661_440
    assert pf == 4 * 32 * 32 * 128 * 32768
    # ragged batch: the sum of the streams' prefixes
    lens = [60000, 70000, 65536]
    w = wl.replace(wl.WORKLOADS["batched_64k"], batch=3)
    pb, pf, _, _ = bench.algorithmic(w, lens)
    assert pf == 4 * 32 * 32 * 128 * sum(lens)
    assert pb == 2 * sum(lens) * 8 * 128 * 2 + 3 * 32 * 32 * 128 * 2 + 3 * 32 * 32 * 129 * 4
    # sparse variant: the selected keys stand in for the prefix (205 chunks of 64)
    _, pf, _, _ = bench.algorithmic(wl.WORKLOADS["text_gqa_128k"], [131072], sparse_tokens=205 * 64)
    assert pf == 4 * 32 * 64 * 128 * 13120


def test_block_bytes_and_flops_by_hand():
    # the 1560-token video block: 4 * Hq * Lb^2 * D flops; Q, K, V, O in bf16 + cache and LSE in fp32
    _, _, bb, bf = bench.algorithmic(wl.WORKLOADS["video_1560"], [31200])
    assert bf == 4 * 12 * 1560 * 1560 * 128
    assert bb == 1560 * 128 * 2 * (12 + 24) + 12 * 1560 * 129 * 4 + 1560 * 12 * 128 * 2


def test_traffic_table_needs_the_same_library_sources(tmp_path):
    shutil.copy(os.path.join(ROOT, "bench.py"), tmp_path / "bench.py")
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "cached_attention_amd" / "csrc"
    src.mkdir(parents=True)
    files = {"fb_kernels.hip": "// kernels v1\n", "fb_api.cpp": "// planner v1\n", "fb_internal.h": "// h v1\n"}
    for name, text in files.items():
        (src / name).write_text(text)
    h = hashlib.sha256()
    for name in ("fb_kernels.hip", "fb_api.cpp", "fb_internal.h"):   # the hash, restated by hand
        h.update(name.encode() + b"\0" + files[name].encode() + b"\0")
    sha = h.hexdigest()[:16]
    (tmp_path / "profiles" / "hbm_traffic.md").write_text(
        "| workload | pass | source | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes |\n"
        "|---|---|---|---|---|---|---|\n"
        f"| text_gqa_128k | prefix | {sha} | `k1` | 1 | 2 | 700000000 |\n"
        f"| text_gqa_128k | prefix | {sha} | `k2` | 1 | 2 | 20000000 |\n"
        f"| text_gqa_128k | block | {sha} | `k3` | 1 | 2 | 5000000 |\n"
        f"| text_gqa_128k~sparse | prefix | {sha} | `k1` | 1 | 2 | 90000000 |\n")
    b2 = _load_bench(str(tmp_path / "bench.py"))
    assert b2.library_source_sha() == sha
    # the prefix pass: the sum of its kernels' rows (split-KV partials + combine)
    assert b2.measured_traffic("text_gqa_128k") == 720000000.0
    assert b2.measured_traffic("text_gqa_128k", "block") == 5000000.0
    assert b2.measured_traffic("text_gqa_128k~sparse") == 90000000.0
    assert b2.measured_traffic("text_mha_32k") is None           # no row for it
    (src / "fb_api.cpp").write_text("// planner v2\n")           # a configuration choice changed since
    assert b2.measured_traffic("text_gqa_128k") is None
    (src / "fb_api.cpp").write_text(files["fb_api.cpp"])
    assert b2.measured_traffic("text_gqa_128k") == 720000000.0
    (src / "fb_kernels.hip").write_text("// kernels v2\n")        # the kernels changed since
    assert b2.measured_traffic("text_gqa_128k") is None


def test_bench_measures_one_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_runs_the_gpu_variant():
    """The oracle baseline times the same variant as the GPU run: fixed period,
    sparse with its own chunk selection, or an adaptive reuse policy."""
    w = wl.ci_version(wl.WORKLOADS["text_gqa_128k"], prefix_len=640, hq=8, hkv=2, block_len=16)
    prefix, blocks = wl.make_inputs(w)
    for variant, kw in [("fixed", {}), ("sparse", {"k_sel": 2}), ("tau", {"tau": 4, "eps": 0.25}),
                        ("gamma", {"gamma": 0.99})]:
        r = bench.cpu_baseline(w, prefix, blocks, 2, budget_s=0.05, variant=variant, **kw)
        assert r["value"] > 0 and r["kind"] == "oracle" and f", {variant}, " in r["sample"]
        # host cores as the OS reports them, and full recompute timed beside the cached block
        assert r["cpu_count"] == os.cpu_count() and r["sched_affinity"] == len(os.sched_getaffinity(0))
        assert r["cores"] >= 1 and r["full_recompute"]["value"] > 0 and r["speedup_vs_full"] > 0
