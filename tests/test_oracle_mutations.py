"""The oracle's pins against planted mistakes in its edge readings (CPU only).

Each case copies the oracle and its pin tests to a scratch directory, changes
one rule in the copy of oracle/rht_oracle.c, and runs the pins on that copy:
they must fail.  The rules are the readings the pages leave to the
implementation and the pins fix ("Random-rotation quantization", "History":
the DRIVE sign code with its scale, and the TurboQuant residual sign code):
the sign bit of an exact zero is +1, a zero row has scale 0, and fp16 values
round to nearest with ties to even.  The repository's own oracle is never
modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("drive sign of an exact zero",
     "put_field(brow, i, 1, h[i] >= 0.0 ? 1u : 0u);", "put_field(brow, i, 1, h[i] > 0.0 ? 1u : 0u);"),
    ("residual sign of an exact zero",
     "put_field(srow, i, 1, ri >= 0.0 ? 1u : 0u);", "put_field(srow, i, 1, ri > 0.0 ? 1u : 0u);"),
    ("unbiased drive scale of a zero row",
     "S = l1 > 0.0 ? ss / l1 : 0.0;", "S = l1 > 0.0 ? ss / l1 : 1.0;"),
    ("biased drive scale of a zero row",
     "S = l1 / d;", "S = l1 > 0.0 ? l1 / d : 1.0;"),
    ("residual scale of a zero row",
     "res_scale[r] = (float)(r1 > 0.0 ? r2 / r1 : 0.0);", "res_scale[r] = (float)(r1 > 0.0 ? r2 / r1 : 1.0);"),
    ("fp16 ties in the normal range",
     "double m = nearbyint(ldexp(f, 11));", "double m = round(ldexp(f, 11));"),
    ("fp16 ties in the subnormal range",
     "double m = nearbyint(ldexp(a, 24));", "double m = round(ldexp(a, 24));"),
]


def scratch_copy(dst):
    os.makedirs(os.path.join(dst, "oracle"))
    for f in ("__init__.py", "rht_oracle.c"):
        shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(dst, "oracle", f))
    os.makedirs(os.path.join(dst, "tests"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))


def run_pins(root):
    env = dict(os.environ, PYTHONPATH=root)
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
                           "-p", "no:cacheprovider"], cwd=root, env=env, capture_output=True, text=True)


def test_unchanged_copy_passes(tmp_path):
    root = str(tmp_path / "copy")
    scratch_copy(root)
    r = run_pins(root)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, what, old, new):
    root = str(tmp_path / "copy")
    scratch_copy(root)
    src = os.path.join(root, "oracle", "rht_oracle.c")
    with open(src) as f:
        text = f.read()
    assert text.count(old) == 1, "the rule to change is not in the oracle as expected: %s" % what
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    r = run_pins(root)
    assert r.returncode != 0, "no pin fails when the oracle gets wrong: %s" % what
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
