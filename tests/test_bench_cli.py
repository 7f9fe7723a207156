"""Host-side checks of bench.py: the one-GPU guard and the counter-summary digest
gate that decides whether a bench line reports measured HBM traffic."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _summary(digest, traffic="123456"):
    return ("# a counter summary\n\n- traffic_bytes_per_launch: " + traffic +
            "\n- source_sha256: `" + digest + "`\n")


def test_traffic_is_reported_only_while_the_digest_matches(tmp_path, monkeypatch):
    b = _bench_module()
    monkeypatch.setattr(b, "PROFILES", str(tmp_path))
    srcs = ("quantize.hip", "common.hpp")
    good = b.source_digest(srcs)
    (tmp_path / "ok.md").write_text(_summary(good))
    (tmp_path / "stale.md").write_text(_summary("0" * 64))
    (tmp_path / "garbled.md").write_text(_summary(good, traffic="n/a"))
    assert b.measured_traffic("ok.md", srcs) == 123456.0
    assert b.measured_traffic("stale.md", srcs) is None        # taken on other kernel sources
    assert b.measured_traffic("garbled.md", srcs) is None
    assert b.measured_traffic("missing.md", srcs) is None
    assert b.source_digest(("gemm_skinny.hip",)) != good       # the digest follows the named sources


def test_committed_counter_summaries_name_their_sources():
    """Each committed counter summary carries a digest in the format the gate reads."""
    b = _bench_module()
    for name in (b.DECODE_COUNTERS, b.QUANT_COUNTERS):
        path = os.path.join(b.PROFILES, name)
        lines = [l for l in open(path) if l.startswith("- source_sha256:")]
        assert len(lines) == 1 and len(lines[0].split("`")[1]) == 64, name
