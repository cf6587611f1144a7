"""Host-side logic of bench.py (no GPU): the one-GPU guard, and the HBM
traffic figure, which is reported only when the committed counter summary
was taken on the current kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_hash_covers_every_kernel_source():
    h = bench.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_hash()


@pytest.fixture
def profile_dir(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    csrc = os.path.join(ROOT, "fp8_block_scaled_02_amd")
    (tmp_path / "fp8_block_scaled_02_amd").symlink_to(csrc)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    return tmp_path / "profiles"


def test_traffic_is_read_only_for_the_current_sources(profile_dir):
    cur = bench.kernel_hash()
    f = profile_dir / "traffic_k.txt"
    f.write_text("# header: ignored\nhbm_bytes_per_launch: 1234567\nkernel_hash: %s\n" % cur)
    assert bench.load_traffic("k") == 1234567
    f.write_text("hbm_bytes_per_launch: 1234567\nkernel_hash: %s\n" % ("0" * 16))
    assert bench.load_traffic("k") is None          # taken on other sources
    f.write_text("kernel_hash: %s\n" % cur)
    assert bench.load_traffic("k") is None          # no figure
    assert bench.load_traffic("missing") is None


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "fp8_block_scaled_02_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// a kernel\n__global__ void k(int* p) { p[0] = 1; }\n")
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    h0 = bench.kernel_hash()
    (csrc / "k.hip").write_text("// the kernel, reworded\n/* and a block\n comment */\n"
                                "__global__ void k(int* p) {   p[0] = 1;  }  // trailing\n")
    assert bench.kernel_hash() == h0
    (csrc / "k.hip").write_text("// a kernel\n__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.kernel_hash() != h0
