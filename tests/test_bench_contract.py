"""CPU checks of bench.py's contract that need no GPU: the one-GPU guard and
the rule that `roofline.traffic` is reported only for the kernel sources the
committed counter summary was taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""              # no JSON line for a refused run


def test_source_hash_ignores_comments_and_spacing(tmp_path):
    src = os.path.join(ROOT, bench.KERNEL_SOURCES[0])
    text = open(src, encoding="utf-8").read()
    a = tmp_path / "a.hip"
    a.write_text(text)
    b = tmp_path / "b.hip"
    b.write_text("// a new header line\n/* and a\n block */\n" + text.replace("\n", "\n\n  "))
    c = tmp_path / "c.hip"
    c.write_text(text + "\nint one_more_symbol;\n")
    ha, hb, hc = (bench.kernel_source_hash([str(p)]) for p in (a, b, c))
    assert ha == hb == bench.kernel_source_hash([src])
    assert hc != ha                            # a code change retires the summary


def _summary(tmp_path, digest, nbytes="1.292860e+10"):
    p = tmp_path / "traffic.md"
    p.write_text(f"HBM bytes per launch (scaled): {nbytes}\n\nkernel source hash: `{digest}`\n")
    return str(p)


def test_traffic_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC",
                        _summary(tmp_path, bench.kernel_source_hash()))
    assert bench.traffic_from_profile() == pytest.approx(1.29286e10)
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", _summary(tmp_path, "0123456789abcdef"))
    assert bench.traffic_from_profile() is None
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "missing.md"))
    assert bench.traffic_from_profile() is None


def test_committed_traffic_summary_parses():
    text = open(bench.PROFILE_TRAFFIC, encoding="utf-8").read()
    assert "kernel source hash:" in text and "HBM bytes per launch (scaled):" in text
