"""Host-side logic of bench.py (no GPU): the one-GPU guard and the rule that a stored HBM
traffic figure is reported only while the kernel's sources are the ones it was measured on."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("args", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_every_gemm_launch_names_existing_sources_and_summary():
    for name, k in bench.KERNELS.items():
        for src in k["sources"]:
            assert os.path.isfile(os.path.join(bench.CSRC, src)), (name, src)
        assert os.path.isfile(os.path.join(ROOT, "profiles", k["traffic"])), name


def test_digest_changes_with_any_source(tmp_path, monkeypatch):
    # a copy of the tree's layout: csrc two levels below the folder that holds include/
    srcs = bench.KERNELS["k_layer_fwd"]["sources"]
    csrc = tmp_path / "pkg" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    for name in srcs:
        dst = os.path.normpath(os.path.join(str(csrc), name))
        with open(dst, "wb") as f:
            f.write(open(os.path.join(bench.CSRC, name), "rb").read())
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    base = bench.csrc_digest(srcs)
    assert bench.csrc_digest(srcs) == base
    for name in srcs:
        p = type(tmp_path)(os.path.normpath(os.path.join(str(csrc), name)))
        orig = p.read_bytes()
        p.write_bytes(orig + b"\n")
        assert bench.csrc_digest(srcs) != base, name
        p.write_bytes(orig)
    assert bench.csrc_digest(srcs) == base


def test_stored_traffic_needs_a_matching_digest(tmp_path, monkeypatch):
    k = bench.KERNELS["k_bwd_gemms<1>"]
    prof = tmp_path / "profiles"
    prof.mkdir()
    digest = bench.csrc_digest(k["sources"])
    (prof / k["traffic"]).write_text(
        f"summary\n\ntraffic_bytes_per_launch: 123456789\ncsrc_digest: {digest}\n")
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    assert bench.stored_traffic("k_bwd_gemms<1>") == 123456789
    (prof / k["traffic"]).write_text(
        "summary\n\ntraffic_bytes_per_launch: 123456789\ncsrc_digest: 0000000000000000\n")
    assert bench.stored_traffic("k_bwd_gemms<1>") is None
    (prof / k["traffic"]).write_text(f"summary\ncsrc_digest: {digest}\n")
    assert bench.stored_traffic("k_bwd_gemms<1>") is None
    (prof / k["traffic"]).unlink()
    assert bench.stored_traffic("k_bwd_gemms<1>") is None
