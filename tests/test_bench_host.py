"""Host-side parts of bench.py: the one-GPU guard, the committed traffic summary lookup and the
CPU baseline record (no GPU needed)."""

import hashlib
import importlib.util
import os
import subprocess
import sys


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def _fake_tree(tmp_path, source, recorded_sha):
    csrc = tmp_path / "attention_backward_fmha_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "kernels_wide.hip").write_bytes(source)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k_bwd_wide_w_deterministic_traffic.txt").write_text(
        "# comment: not a field\nkernel_source_sha256: %s\nmode: deterministic\n"
        "read_bytes_per_launch: 1000\nwrite_bytes_per_launch: 234\n" % recorded_sha)


def test_traffic_is_read_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    b = _bench()
    source = b"// kernel source\n"
    _fake_tree(tmp_path, source, hashlib.sha256(source).hexdigest())
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("k_bwd_wide", "w", "deterministic") == 1234
    assert b.measured_traffic("k_bwd_wide", "w", "atomic") is None  # no summary for that mode
    assert b.measured_traffic("k_bwd_main", "w", "deterministic") is None  # another kernel
    (tmp_path / "attention_backward_fmha_amd" / "csrc" / "kernels_wide.hip").write_bytes(source + b"// edited\n")
    assert b.measured_traffic("k_bwd_wide", "w", "deterministic") is None  # the kernel changed since


def test_committed_traffic_summaries_are_well_formed():
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith("_traffic.txt")]
    assert names, "no traffic summary committed"
    for n in names:
        fields = dict(line.split(":", 1) for line in open(os.path.join(prof, n))
                      if ":" in line and not line.startswith("#"))
        assert len(fields["kernel_source_sha256"].strip()) == 64
        assert fields["mode"].strip() in ("deterministic", "atomic", "atomic16")
        assert int(fields["read_bytes_per_launch"]) > 0 and int(fields["write_bytes_per_launch"]) > 0


def test_cpu_baseline_record():
    b = _bench()
    from attention_backward_fmha_amd import inputs as I
    w = dict(I.WORKLOADS["tiny"])
    rec = b.cpu_baseline(w, 0.05)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "repetitions" in rec["sample"]
