"""Planted mistakes: the oracle's pins have power (CPU only).

Each case below is one plausible slip in one oracle function -- a transposed
operand, a wrong constant or divisor, a dropped term, the other tie rule, the
other bit or byte order -- written as a text substitution of one line of the
oracle's source. The oracle package is copied to a temporary directory with
the substitution applied, and the pin tests that cover that function run on
the copy in a child process: at least one of them must fail. A mutant that
breaks the import or collection instead does not count as caught.

The substitutions name exact source lines, so a case fails loudly (its
pattern no longer occurs once) if the oracle is rewritten; update the case
with the rewrite.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCORE_PINS = ["tests/test_oracle_score.py"]
COMPRESS_PINS = ["tests/test_oracle_compress.py"]
PACK_PINS = ["tests/test_oracle_pack.py"]
CODEBOOK_PINS = ["tests/test_oracle_codebook.py"]
MSE_PINS = ["tests/test_oracle_mse.py"]
SPLIT_PINS = ["tests/test_oracle_split.py"]
ATTEND_PINS = ["tests/test_oracle_attend.py"]

# (case, oracle file, text in it, replacement, pin test files)
MUTATIONS = [
    ("Pi not transposed in the reconstruction", "oracle/score.py",
     "mse_part = c @ np.asarray(Pi, np.float64)", "mse_part = c @ np.asarray(Pi, np.float64).T", SCORE_PINS),
    ("S_mat not transposed in the reconstruction", "oracle/score.py",
     "qjl_part = sig @ np.asarray(S_mat, np.float64)", "qjl_part = sig @ np.asarray(S_mat, np.float64).T",
     SCORE_PINS),
    ("constant sqrt(2/pi) for sqrt(pi/2)", "oracle/score.py",
     "math.sqrt(math.pi / 2.0)", "math.sqrt(2.0 / math.pi)", SCORE_PINS),
    ("QJL divisor sqrt(D) for D", "oracle/score.py",
     "(QJL_SQRT_HALF_PI / D) * g * qjl_part", "(QJL_SQRT_HALF_PI / D**0.5) * g * qjl_part", SCORE_PINS),
    ("gamma dropped from the transformed scores", "oracle/score.py",
     "out[:, s0:s1] = mse + (QJL_SQRT_HALF_PI / D) * g * res", "out[:, s0:s1] = mse + (QJL_SQRT_HALF_PI / D) * res",
     SCORE_PINS),
    ("A = Pi^T q", "oracle/query_transform.py",
     "A = q64 @ np.asarray(Pi, np.float64).T", "A = q64 @ np.asarray(Pi, np.float64)", SCORE_PINS),
    ("compressor rotates with Pi^T", "oracle/compress.py",
     "return np.asarray(keys, np.float64) @ np.asarray(Pi, np.float64).T",
     "return np.asarray(keys, np.float64) @ np.asarray(Pi, np.float64)", COMPRESS_PINS),
    ("compressor signs of S^T r", "oracle/compress.py",
     "proj = r @ np.asarray(S_mat, np.float64).T", "proj = r @ np.asarray(S_mat, np.float64)", COMPRESS_PINS),
    ("keys compressed without normalising", "oracle/compress.py",
     "unit = k / np.where(norm > 0.0, norm, 1.0)[:, None]", "unit = k", COMPRESS_PINS),
    ("ties take the upper index", "oracle/compress.py",
     'side="left").astype(np.uint8)', 'side="right").astype(np.uint8)', COMPRESS_PINS),
    ("Gaussian law with variance 2/d", "oracle/codebook.py",
     "np.exp(-0.5 * d * x * x)", "np.exp(-0.25 * d * x * x)", CODEBOOK_PINS),
    ("sphere law exponent (d-2)/2", "oracle/codebook.py",
     "** ((d - 3) / 2.0)", "** ((d - 2) / 2.0)", CODEBOOK_PINS),
    ("MSB-first index bytes", "oracle/pack.py",
     'return np.packbits(stream, axis=-1, bitorder="little")', 'return np.packbits(stream, axis=-1, bitorder="big")',
     PACK_PINS),
    ("sign bit polarity flipped", "oracle/pack.py",
     "return np.packbits(sign > 0, axis=-1", "return np.packbits(sign < 0, axis=-1", PACK_PINS),
    ("bit order reversed inside an index", "oracle/pack.py",
     "planes = (idx[..., :, None] >> np.arange(bits, dtype=np.uint8)) & 1",
     "planes = (idx[..., :, None] >> np.arange(bits, dtype=np.uint8)[::-1]) & 1", PACK_PINS),
]


def _copy_tree(dst: str, pins: list[str]) -> None:
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(dst, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    for f in ["tests/conftest.py", *pins]:
        shutil.copy(os.path.join(ROOT, f), os.path.join(dst, f))


@pytest.mark.parametrize("case,path,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, case, path, old, new, pins):
    dst = str(tmp_path)
    _copy_tree(dst, pins)
    target = os.path.join(dst, path)
    with open(target) as f:
        src = f.read()
    assert src.count(old) == 1, f"{case}: the line to mutate no longer occurs once in {path}"
    with open(target, "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          *pins], cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    tail = "\n".join((res.stdout + res.stderr).splitlines()[-15:])
    assert res.returncode != 0, f"{case}: every pin passed on the mutant\n{tail}"
    assert res.returncode == 1, f"{case}: the mutant did not run as a test failure (rc {res.returncode})\n{tail}"
