"""Host-side logic of bench.py, without a GPU.

The benchmark measures one GPU only: any other --gpus value ends with a JSON line that says so and
exit status 2, before any device work. Unknown section names are refused the same way. Counter-derived
figures (HBM traffic, MFMA utilisation) are reported only while the kernel sources they were taken on
still hash, comments and whitespace aside, to the recorded value.
"""

import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_json_line():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2, r.stderr
        line = json.loads(r.stdout.strip().splitlines()[-1])
        assert line["n_gpus"] == int(n) and "one GPU" in line["error"]


def test_unknown_sections_are_refused():
    r = _run("--only", "gemv,nosuchsection")
    assert r.returncode != 0
    assert "nosuchsection" in r.stderr


def test_sources_hash_ignores_comments_and_whitespace(tmp_path):
    b = _bench()
    a = tmp_path / "a.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    c.write_text("/* header */ int f(int x)\n{ return x + 1; }\n")
    b.ROOT = str(tmp_path)
    assert b.sources_sha256(["a.hip"]) == b.sources_sha256(["c.hip"])
    c.write_text("int f(int x) { return x + 2; }\n")
    assert b.sources_sha256(["a.hip"]) != b.sources_sha256(["c.hip"])


def test_counter_figures_follow_their_sources(tmp_path):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    b.ROOT = str(tmp_path)
    b.MEASURED["probe"] = {"sources": ("k.hip",), "sha256": b.sources_sha256(["k.hip"]), "value": 123}
    assert b.measured("probe") == 123
    src.write_text("__global__ void k() { int a = 0; (void)a; }\n")
    assert b.measured("probe") is None
    b.MEASURED["probe"]["sha256"] = None
    assert b.measured("probe") is None


def test_recorded_counter_figures_name_existing_sources():
    b = _bench()
    for key, m in b.MEASURED.items():
        for rel in m["sources"]:
            assert os.path.isfile(os.path.join(ROOT, rel)), (key, rel)
        assert m["sha256"] is None or len(m["sha256"]) == 64, key
