"""Host-side pieces of bench.py: the code hash that ties committed counter records to the kernel
code they were taken on, the records themselves, and the one-GPU rule."""
import glob
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_strip_comments_keeps_code_and_literals(bench):
    src = ('int a = 1; // trailing\n'
           '/* block\n   comment */ const char* s = "//not a comment /* nor this */";\n'
           "char c = '\\''; char d = '/';\n"
           '\n   \n'
           'int b = a /* inline */ + 2;   \n')
    assert bench.strip_comments(src) == (
        'int a = 1;\n'
        ' const char* s = "//not a comment /* nor this */";\n'
        "char c = '\\''; char d = '/';\n"
        'int b = a  + 2;')


def test_code_hash_ignores_comments_only(bench):
    code = "__global__ void k(int* p) {\n  p[0] = 1;\n}\n"
    h = lambda t: bench.strip_comments(t)
    assert h(code) == h("// header\n" + code.replace("{\n", "{  // body\n") + "\n/* end */\n")
    assert h(code) != h(code.replace("p[0] = 1", "p[0] = 2"))
    assert h(code) != h(code.replace("p[0]", "p[1]"))


def test_traffic_records_match_current_code(bench):
    recs = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.json")))
    assert recs, "no committed counter records"
    for path in recs:
        r = json.load(open(path))
        for key in ("workload", "kernel", "source", "code_sha256", "bytes_per_launch",
                    "algorithmic_bytes_per_launch", "fetch_scale", "write_scale", "commands"):
            assert key in r, f"{os.path.basename(path)}: missing {key}"
        # the scales come from a copy of known size: fetch counts half the bytes, write all
        assert 1.9 < r["fetch_scale"] < 2.1 and 0.95 < r["write_scale"] < 1.05, path
        # HBM traffic cannot be far below what the kernel must move
        assert r["bytes_per_launch"] >= 0.95 * r["algorithmic_bytes_per_launch"], path
        if r["code_sha256"] == bench.code_sha256(r["source"]):
            op = "copy_blocks" if r["source"] == "block_copy.hip" else "paged_attention"
            assert bench.traffic_from_profile(r["workload"], op, r["source"]) == r["bytes_per_launch"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_clock_record(bench):
    """The prefill kernel's counter record: MFMA busy is a fraction, the clock sits below the
    2.4 GHz the dense-peak figure assumes, and the bench returns it only on the current code."""
    path = os.path.join(ROOT, "profiles", "prefill_kernel_mfma_busy.json")
    r = json.load(open(path))
    assert r["workloads"]
    for w, v in r["workloads"].items():
        assert 0 < v["mfma_busy"] < 1 and 1.0 < v["clock_ghz"] <= 2.45, (w, v)
        got = bench.clock_from_profile(w)
        assert got == (v if r["code_sha256"] == bench.code_sha256(r["source"]) else None)
