"""Host-side parts of bench.py that run without a GPU: the single-GPU
refusal and the rule that a committed HBM-traffic figure is used only while
the kernel source it was measured on is unchanged."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILE = "w4a4_gemm_prefill_32768x10240x5120_traffic.md"


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
    r = _run_bench(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def _fake_tree(tmp_path, kernel_text):
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "nvfp4_w4a4_quantized_03_amd" / "csrc"
    csrc.mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "profiles", PROFILE), tmp_path / "profiles" / PROFILE)
    (csrc / "gemm.hip").write_bytes(kernel_text)


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    text = open(os.path.join(ROOT, "profiles", PROFILE)).read()
    want = float(text.split("hbm_bytes_per_launch:")[1].split()[0])
    sha = text.split("source_sha256_16:")[1].split()[0]
    src = open(os.path.join(ROOT, "nvfp4_w4a4_quantized_03_amd", "csrc", "gemm.hip"), "rb").read()
    # the committed source, if it is the profiled one, gives the figure
    _fake_tree(tmp_path, src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.measured_traffic(PROFILE, 1)
    if bench.source_hash("gemm.hip") == sha:
        assert got == want
    else:
        assert got is None
    # any change to the source withdraws it
    (tmp_path / "nvfp4_w4a4_quantized_03_amd" / "csrc" / "gemm.hip").write_bytes(src + b"\n")
    assert bench.measured_traffic(PROFILE, 1) is None
    # and a missing summary gives none
    os.remove(tmp_path / "profiles" / PROFILE)
    assert bench.measured_traffic(PROFILE, 1) is None
