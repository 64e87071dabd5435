"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every library source is compiled with the sanitizers on its host pass (device
code is built as usual and never run), linked with tests/abi_sanitize.cpp,
and run on the CPU: argument validation, empty calls, misaligned pointers and
the pure size and name queries, at the int32 and int64 extremes. Any memory
error or undefined behaviour (signed overflow in a size computation, say)
fails the run. Build products go to a temporary directory.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_attention_scoring_amd", "csrc")
def _library_sources():
    """The .hip sources the library build compiles (its SOURCES list)."""
    import ast
    with open(os.path.join(ROOT, "compressed_attention_scoring_amd", "build.py")) as f:
        tree = ast.parse(f.read())
    for node in tree.body:
        if isinstance(node, ast.Assign) and any(getattr(t, "id", None) == "SOURCES" for t in node.targets):
            return [os.path.splitext(s)[0] for s in ast.literal_eval(node.value)]
    raise AssertionError("build.py has no SOURCES list")


SOURCES = _library_sources()
SANITIZERS = ["address", "undefined"]
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _host_only(flag_list):
    """Each sanitizer flag applies to the host pass only."""
    out = []
    for f in flag_list:
        out += ["-Xarch_host", f]
    return out


@pytest.mark.slow
def test_abi_under_host_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    san = [f"-fsanitize={s}" for s in SANITIZERS] + ["-fno-sanitize-recover=all"]
    common = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    device = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    procs, objs = [], []
    for name in SOURCES:
        obj = str(tmp_path / f"{name}.o")
        cmd = [HIPCC, *device, *common, *_host_only(san), "-c", os.path.join(CSRC, f"{name}.hip"), "-o", obj]
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for name, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"{name}.hip failed to build:\n{out[-4000:]}"
    driver = str(tmp_path / "driver.o")
    subprocess.run([CLANG, *common, *san, "-c", os.path.join(ROOT, "tests", "abi_sanitize.cpp"), "-o", driver],
                   check=True)
    exe = str(tmp_path / "abi_san")
    subprocess.run([CLANG, *san, driver, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "0 failures" in res.stdout
    assert "runtime error" not in res.stderr
