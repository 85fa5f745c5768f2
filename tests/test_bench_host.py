"""Host-side logic of bench.py (CPU only): the one-GPU rule and the lookup
of stored counter figures, which must be used only for the kernel sources
they were measured on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write_summary(root, digest, nbytes):
    os.makedirs(os.path.join(root, "profiles"))
    with open(os.path.join(root, "profiles", "main_kernel_wl_traffic.md"), "w") as f:
        f.write("# summary\n\ntext\n\n- kernel: main_kernel\n"
                f"- bytes per launch: {nbytes}\n- source digest: `{digest}`\n")


def test_stored_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "0123456789abcdef")
    assert bench.stored_traffic("wl", "main_kernel") is None          # no summary
    _write_summary(str(tmp_path), "0123456789abcdef", 36245113)
    assert bench.stored_traffic("wl", "main_kernel") == 36245113
    monkeypatch.setattr(bench, "source_digest", lambda: "fedcba9876543210")
    assert bench.stored_traffic("wl", "main_kernel") is None          # sources changed


def test_source_digest_covers_the_kernel_sources():
    d = bench.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert d == bench.source_digest()
