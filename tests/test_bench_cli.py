"""Host-side checks of bench.py's command line: the default warm-up and timed
step counts per workload, explicit values taken as given, and the one-GPU
guard."""
import subprocess
import sys

import pytest

import bench


def _parse(argv, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", *argv])
    return bench.parse()


@pytest.mark.parametrize("workload,steps,warmup", [(3, 300, 200), (6, 300, 200), (7, 300, 200), (5, 50, 10)])
def test_default_steps_per_workload(workload, steps, warmup, monkeypatch):
    a = _parse(["--workload", str(workload)], monkeypatch)
    assert (a.steps, a.warmup) == (steps, warmup)


def test_explicit_steps_are_used_as_given(monkeypatch):
    a = _parse(["--steps", "7", "--warmup", "0"], monkeypatch)
    assert (a.steps, a.warmup, a.gpus, a.workload) == (7, 0, 1, 3)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.os.path.dirname(bench.os.path.abspath(bench.__file__)), timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


@pytest.mark.parametrize("split_name,q_len,fp8", [("mla_decode_split", 1, False), ("mla_decode_split", 2, False),
                                                  ("mla_decode8_split", 1, True)])
def test_decode_traffic_summaries_are_found_under_the_names_the_bench_builds(split_name, q_len, fp8):
    name = bench.split_traffic_name(split_name, 64, q_len, 128, 8192, fp8)
    assert bench.os.path.exists(bench.os.path.join(bench.PROFILES, f"{name}_hbm_traffic.md")), name


def test_traffic_summaries_of_the_smaller_and_ragged_decodes_are_found():
    # workload 2 (B=16, H=16, L=4096) and workload 4 (B=32, H=128, contexts
    # drawn on [1024, 32768] with seed 1504: the longest is 31044)
    from synth import make_ragged_lens
    lens = make_ragged_lens(1504, 32, 1024, 32768)
    for b, h, L in ((16, 16, 4096), (32, 128, int(max(lens)))):
        name = bench.split_traffic_name("mla_decode_split", b, 1, h, L, False)
        assert bench.os.path.exists(bench.os.path.join(bench.PROFILES, f"{name}_hbm_traffic.md")), name


def test_prefill_traffic_summary_is_found_under_the_name_the_bench_builds():
    assert bench.os.path.exists(bench.os.path.join(bench.PROFILES, "mla_prefill_attn_B4_S4096_H128_hbm_traffic.md"))
