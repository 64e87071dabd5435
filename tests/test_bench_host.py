"""Host logic of bench.py that needs no GPU: the source digest that keys the
committed profile records to the code they were taken on."""
import glob
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _digest_of(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    old = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        return bench.source_digest([name])
    finally:
        bench.ROOT = old


BASE = 'int f(int x) {\n    return x + 1;\n}\nconst char* s = "a//b";\n'


def test_digest_ignores_comments_and_blank_lines(tmp_path):
    d0 = _digest_of(tmp_path, "a.hip", BASE)
    edited = ("// header\n/* block\n   comment */\nint f(int x) {  // trailing\n\n"
              "    return x + 1;   \n}\nconst char* s = \"a//b\"; /* end */\n")
    assert _digest_of(tmp_path, "b.hip", edited) == d0


def test_digest_sees_code_changes(tmp_path):
    d0 = _digest_of(tmp_path, "a.hip", BASE)
    assert _digest_of(tmp_path, "b.hip", BASE.replace("x + 1", "x + 2")) != d0
    # a comment marker inside a string literal is code
    assert _digest_of(tmp_path, "c.hip", BASE.replace('"a//b"', '"a//c"')) != d0
    # character literals with escapes do not swallow what follows
    assert (_digest_of(tmp_path, "d.hip", BASE + "char q = '\\'';\nint y = 1;\n")
            != _digest_of(tmp_path, "e.hip", BASE + "char q = '\\'';\nint y = 2;\n"))


def test_records_name_existing_sources():
    recs = glob.glob(os.path.join(ROOT, "profiles", "*.json"))
    assert recs
    for p in recs:
        with open(p) as f:
            rec = json.load(f)
        assert rec["source_files"], p
        for s in rec["source_files"]:
            assert os.path.isfile(os.path.join(ROOT, s)), (p, s)
        assert len(rec["source_sha256"]) == 64, p


def test_more_than_one_gpu_is_refused():
    """--gpus N with N > 1 prints why and exits before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["n_gpus"] == 2 and "one GPU" in d["error"]
