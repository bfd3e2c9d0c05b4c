"""CPU checks of bench.py's contract that need no GPU: the one-GPU refusal of
--gpus N > 1, and the HBM-traffic figure it takes from the committed counter
summary only while the attention kernel's code matches the summary's digest."""

import importlib.util
import json
import os
import subprocess
import sys

from segment_autoregressive_dit_amd.profile_workload import source_digest

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


def test_source_digest_ignores_comments_only(tmp_path):
    path = os.path.join(ROOT, "segment_autoregressive_dit_amd", "csrc", "attention.hip")
    src = open(path).read()
    tmp = tmp_path / "probe.hip"
    tmp.write_text("// an added comment line\n" + src.replace("namespace nomas {", "namespace nomas {  /* note */", 1))
    assert source_digest(str(tmp)) == source_digest(path)
    tmp.write_text(src.replace("constexpr float kTau = 8.0f;", "constexpr float kTau = 7.0f;", 1))
    assert source_digest(str(tmp)) != source_digest(path)


def test_traffic_comes_from_a_matching_summary_only(tmp_path):
    bench = _bench_module()
    summary = json.load(open(bench.PMC_SUMMARY))
    assert summary["source"] == "attention.hip"
    # the figure is reported exactly when the summary was taken from the kernel
    # as it stands (otherwise null until the counters are taken again)
    if summary["source_digest"] == source_digest(bench.ATTN_SRC):
        assert bench.traffic_per_launch() == summary["hbm_bytes_per_launch"]
    else:
        assert bench.traffic_per_launch() is None
    # a summary of this very code yields its figure
    same = dict(summary, source_digest=source_digest(bench.ATTN_SRC))
    p0 = tmp_path / "same.json"
    p0.write_text(json.dumps(same))
    bench.PMC_SUMMARY = str(p0)
    assert bench.traffic_per_launch() == summary["hbm_bytes_per_launch"]
    # a summary of other code yields no figure
    other = dict(summary, source_digest="0" * 64)
    p = tmp_path / "summary.json"
    p.write_text(json.dumps(other))
    bench.PMC_SUMMARY = str(p)
    assert bench.traffic_per_launch() is None
