"""CPU: bench.py's host logic -- the one-GPU contract, the algorithmic-byte
count the bench line divides by, and the traffic figures that apply only
to the kernel sources they were measured with."""
import os
import subprocess
import sys

import numpy as np

from tests.conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no bench line


def test_touched_bytes_per_expert():
    """Per touched expert: packed E2M1 codes (half a byte per weight) plus
    one E8M0 byte per 32 weights, gate_up [2I, H] and down [H, I]; experts
    with no token cost nothing.  c2's shapes give 13.37 + 6.68 MB."""
    H, I = 6144, 2048
    counts = np.array([0, 3, 0, 1, 5], np.int32)
    gu, dn = bench.touched_bytes(counts, H, I)
    per_gu = 2 * I * H // 2 + 2 * I * H // 32
    per_dn = H * I // 2 + H * I // 32
    assert (gu, dn) == (3 * per_gu, 3 * per_dn)
    assert per_gu == 13_369_344 and per_dn == 6_684_672
    assert bench.touched_bytes(np.zeros(8, np.int32), H, I) == (0, 0)


def test_traffic_applies_only_to_the_sources_it_was_measured_with(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    (csrc / "a.hip").write_text("kernel one\n")
    (csrc / "b.h").write_text("header\n")
    (csrc / "notes.txt").write_text("not a source\n")
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    sha = bench.sources_sha256()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.txt").write_text(
        "# comment line\n"
        f"wl_a gate_kernel {sha} 12345\n"
        f"wl_a other_kernel {sha} 999\n"
        "wl_b gate_kernel 0123abcd 777\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl_a", "gate_kernel") == 12345
    assert bench.measured_traffic("wl_a", "other_kernel") == 999
    assert bench.measured_traffic("wl_b", "gate_kernel") is None  # other sources
    assert bench.measured_traffic("wl_c", "gate_kernel") is None  # not measured
    (csrc / "notes.txt").write_text("edited notes change nothing\n")
    assert bench.sources_sha256() == sha
    (csrc / "a.hip").write_text("kernel two\n")  # any kernel edit voids the figures
    assert bench.sources_sha256() != sha
    assert bench.measured_traffic("wl_a", "gate_kernel") is None


def test_committed_traffic_file_is_well_formed():
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert rows
    for r in rows:
        assert len(r) == 4 and len(r[2]) == 64 and int(r[3]) > 0
