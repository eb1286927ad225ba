"""Host-side checks of bench.py's command line (no GPU is touched)."""
import os
import subprocess
import sys

from conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
    assert not r.stdout.lstrip().startswith("{")   # no result line


def test_bench_refuses_a_multi_rank_launch():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=300, cwd=ROOT, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def _profile_fields(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_recorded_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    import shutil
    import bench
    name = "gemm_decode_kernel_M16_L128_traffic.txt"
    kv = _profile_fields(os.path.join(ROOT, "profiles", name))
    # the summary's own arithmetic: each counter scaled by what it reads for the plain copy of
    # known size, KiB per dispatch -> bytes per launch
    copy = float(kv["copy_bytes_per_dispatch"])
    f_scale = copy / (1024 * float(kv["copy_fetch_kib_per_dispatch"]))
    w_scale = copy / (1024 * float(kv["copy_write_kib_per_dispatch"]))
    assert abs(f_scale - float(kv["fetch_scale"])) < 1e-4 and abs(w_scale - float(kv["write_scale"])) < 1e-4
    expect = 1024 * (float(kv["fetch_kib_per_dispatch"]) * f_scale +
                     float(kv["write_kib_per_dispatch"]) * w_scale)
    assert abs(expect - float(kv["traffic_bytes_per_launch"])) <= 1024
    # reported only while the kernel's sources are the ones it was taken on
    got = bench.recorded_traffic("gemm_decode_kernel", "M16_L128")
    if kv["source_digest"] == bench.source_digest("gemm_decode_kernel"):
        assert got == float(kv["traffic_bytes_per_launch"])
    else:
        assert got is None
    # a copy of the tree whose kernel source differs: no traffic figure
    csrc = tmp_path / "ternary_weight_bit_bitlinear_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("gemm_decode.hip", "common.h"):
        shutil.copy(os.path.join(ROOT, "ternary_weight_bit_bitlinear_amd", "csrc", f), csrc / f)
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", name), tmp_path / "profiles" / name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("gemm_decode_kernel", "M16_L128") == got
    with open(csrc / "gemm_decode.hip", "a") as fh:
        fh.write("\n// changed\n")
    assert bench.recorded_traffic("gemm_decode_kernel", "M16_L128") is None
    assert bench.recorded_traffic("gemm_decode_kernel", "M4_L128") is None   # no summary
