"""Host logic of bench.py that runs without a GPU: the one-GPU rule, the
hash of the kernel sources that gates the measured traffic, and the gate
itself against the committed counter summaries."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    """A comment or a reflowed line leaves the hash alone; a changed token
    does not."""
    csrc = tmp_path / "log_mel_spectrogram_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = csrc / "k.hip"
    py = csrc / "g.py"

    def h(hip, gen):
        src.write_text(hip)
        py.write_text(gen)
        return bench.kernel_source_hash(("k.hip", "g.py"))

    base = h("int f(int a) { return a + 1; }\n", "X = 1\n")
    assert h("// note\nint f(int a) {\n  return a + 1;  /* one */\n}\n",
             '"""doc"""\nX = 1  # the value\n') == base
    assert h("int f(int a) { return a + 2; }\n", "X = 1\n") != base
    assert h("int f(int a) { return a + 1; }\n", "X = 2\n") != base


def _traffic_record(profile):
    rec = None
    with open(os.path.join(ROOT, "profiles", f"{profile}_pmc.md")) as fh:
        for line in fh:
            if line.startswith("TRAFFIC_JSON "):
                rec = json.loads(line[len("TRAFFIC_JSON "):])
    return rec


@pytest.mark.parametrize("profile,files", [("logmel_tiles_c2", bench.TILES_SOURCES),
                                           ("logmel_tiles_c4", bench.TILES_SOURCES),
                                           ("logmel_resample_c2_44k", bench.RESAMPLE_SOURCES)])
def test_traffic_gate_follows_the_source_hash(profile, files, monkeypatch):
    """The committed summary's bytes are read back exactly when its hash is
    the sources' hash, and never for another hash. Its bytes are the two
    counters' per-dispatch means scaled by the copy calibration (fetch x 2,
    write x 1, KiB); the record keeps the means rounded to whole KiB."""
    rec = _traffic_record(profile)
    assert rec is not None
    from_kib = 1024 * (rec["fetch_scale"] * rec["fetch_kib"] + rec["write_scale"] * rec["write_kib"])
    assert abs(rec["hbm_bytes_per_launch"] - from_kib) <= 512 * (rec["fetch_scale"] +
                                                                 rec["write_scale"])
    got = bench.measured_traffic(profile, files)
    if rec["kernel_source_hash"] == bench.kernel_source_hash(files):
        assert got == rec["hbm_bytes_per_launch"]
    else:
        assert got is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: "0" * 16)
    assert bench.measured_traffic(profile, files) is None
    assert bench.measured_traffic("no_such_profile", files) is None
