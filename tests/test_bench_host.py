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


def test_work_matches_the_algorithmic_counts():
    """The headline's algorithmic work: L1 pairs B*H*(2 N m + m^2)*d (maps
    and A), 4 m^3 iters per head for Newton-Schulz, 2 m N d for K_LK V."""
    from nystr_linear_attention_amd import workloads as wl
    w = wl.HEADLINE
    wk = bench.work(w)
    assert wk["map_pairs"] + wk["amat_pairs"] == 8 * (2 * 3136 * 49 + 49 * 49) * 64 == 158581248
    assert wk["ns"] == 8 * 4 * 49 ** 3 * 20
    assert wk["klkv"] == 8 * 2 * 49 * 3136 * 64
    g = bench.work(wl.BY_NAME["gauss_f32_b16h2_n3136_d64_m49_qk"])
    assert g["map_pairs"] == 32 * 3136 * 49 * 64      # K = Q: one map


def test_host_info_names_cpu_and_blas():
    info = bench.host_info()
    assert info["usable_cores"] >= 1
    assert isinstance(info["blas"], list)
