"""The benchmark's command-line contract.

`bench.py` prints one JSON line: the throughput of the four calls over one
synthetic batch (tokens/s), the step time, the roofline entry of the dominant
kernel (achieved = algorithmic work / its time), and, unless disabled, the
oracle's throughput on the host and the hash check against it.  More than one
GPU is refused before any GPU work.  Each run here is a child process of its own.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None, timeout=240):
    e = dict(os.environ)
    e.update(env or {})
    print("bench.py " + " ".join(args), flush=True)
    return subprocess.run([sys.executable, "bench.py", *args], cwd=ROOT, env=e,
                          capture_output=True, text=True, timeout=timeout)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      (["--gpus", "1"], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(*args, env=env, timeout=120)
    assert r.returncode == 2, r.stderr[-2000:]
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _record(stdout):
    lines = [ln for ln in stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, stdout[-2000:]
    return json.loads(lines[0])


def _check_common(rec, steps, warmup):
    assert rec["unit"] == "tokens/s" and rec["n_gpus"] == 1
    assert rec["steps"] == steps and rec["warmup"] == warmup
    assert rec["higher_is_better"] is True and rec["scaling"] == "weak"
    assert rec["vs_baseline"] is None
    assert rec["dtype"] == "bf16" and rec["data"] == "synthetic"
    cfg = rec["config"]
    assert cfg["workload"] == "short_4k"
    tokens = cfg["batch"] * cfg["seq_len"]
    assert rec["ms_per_step"] > 0
    # value is the step's throughput: the tokens of one batch over the step time
    # (ms_per_step is printed to 4 decimals, value to 0.1 token/s)
    ms = rec["ms_per_step"]
    assert tokens / ((ms + 5e-5) * 1e-3) - 0.1 <= rec["value"] <= tokens / ((ms - 5e-5) * 1e-3) + 0.1
    roof = rec["roofline"]
    assert set(roof) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert roof["bound"] in ("hbm", "mfma")
    assert roof["unit"] == ("GB/s" if roof["bound"] == "hbm" else "TFLOP/s")
    assert roof["peak"] == (8000.0 if roof["bound"] == "hbm" else 2500.0)
    assert 0 < roof["frac"] < 1
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-2)
    assert set(rec["kernels"]) == {"lsh_hash", "lsh_sort", "lsh_chunk_attn", "lsh_combine_rounds"}
    for e in rec["kernels"].values():
        assert e["ms"] > 0 and 0 <= e["mfma_frac"] < 1 and 0 <= e["hbm_frac"] < 1


@pytest.mark.gpu
def test_bench_line_with_cpu_baseline():
    r = _run("--workload", "short_4k", "--steps", "3", "--warmup", "2")
    assert r.returncode == 0, r.stderr[-3000:]
    rec = _record(r.stdout)
    _check_common(rec, 3, 2)
    base = rec["cpu_baseline"]
    assert base["kind"] == "oracle" and base["unit"] == "tokens/s"
    assert base["value"] > 0 and base["cores"] >= 1 and base["sample"]
    hc = rec["hash_check"]
    assert hc["hashes"] > 0
    assert hc["mismatches_beyond_near_ties"] == 0
    assert hc["mismatches"] <= hc["near_ties"]


@pytest.mark.gpu
def test_bench_line_graph_replay():
    r = _run("--workload", "short_4k", "--steps", "3", "--warmup", "2", "--graph", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-3000:]
    rec = _record(r.stdout)
    _check_common(rec, 3, 2)
    assert rec["config"]["graph"] is True and rec["config"]["eager_ms_per_step"] > 0
    assert "cpu_baseline" not in rec
