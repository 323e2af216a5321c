"""The oracle's pins against planted mistakes (CPU only).

Each case copies the oracle and its pin tests to a scratch directory, changes
one rule in the copy of oracle/rht_oracle.c, and runs the pins on that copy:
they must fail.  The repository's own oracle is never modified.

Two groups of mistakes:
  * the readings the pages leave to the implementation and the pins fix
    ("Random-rotation quantization", "History": the DRIVE sign code with its
    scale, and the TurboQuant residual sign code): the sign bit of an exact
    zero is +1, a zero row has scale 0, and fp16 values round to nearest with
    ties to even;
  * plausible slips anywhere in the arithmetic: a butterfly sign, the sign
    generator, a dropped or wrong normalization in an encoder, decoder, scale
    or score, the inverse rotation's signs, attention's scale and
    normalization, the fp16 codec's exponents and overflow point, the
    Lloyd-Max centroid, the Jacobian of the finite-d marginal, and the bit
    order of the packed codes.

The copies run concurrently (each is an independent pytest process).
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what, [(text in oracle/rht_oracle.c, replacement, which occurrence)])
MUTATIONS = [
    ("drive sign of an exact zero",
     [("put_field(brow, i, 1, h[i] >= 0.0 ? 1u : 0u);", "put_field(brow, i, 1, h[i] > 0.0 ? 1u : 0u);", 0)]),
    ("residual sign of an exact zero",
     [("put_field(srow, i, 1, ri >= 0.0 ? 1u : 0u);", "put_field(srow, i, 1, ri > 0.0 ? 1u : 0u);", 0)]),
    ("unbiased drive scale of a zero row",
     [("S = l1 > 0.0 ? ss / l1 : 0.0;", "S = l1 > 0.0 ? ss / l1 : 1.0;", 0)]),
    ("biased drive scale of a zero row",
     [("S = l1 / d;", "S = l1 > 0.0 ? l1 / d : 1.0;", 0)]),
    ("residual scale of a zero row",
     [("res_scale[r] = (float)(r1 > 0.0 ? r2 / r1 : 0.0);", "res_scale[r] = (float)(r1 > 0.0 ? r2 / r1 : 1.0);", 0)]),
    ("fp16 ties in the normal range",
     [("double m = nearbyint(ldexp(f, 11));", "double m = round(ldexp(f, 11));", 0)]),
    ("fp16 ties in the subnormal range",
     [("double m = nearbyint(ldexp(a, 24));", "double m = round(ldexp(a, 24));", 0)]),
    ("fwht butterfly sign",
     [("v[j + h] = a - b;", "v[j + h] = b - a;", 0)]),
    ("sign taken from another bit of the generator output",
     [("s[i] = (r >> 63) ? (int8_t)-1 : (int8_t)1;", "s[i] = ((r >> 62) & 1) ? (int8_t)-1 : (int8_t)1;", 0)]),
    ("splitmix64 shift",
     [("z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;", "z = (z ^ (z >> 28)) * 0x94D049BB133111EBULL;", 0)]),
    ("mse encoder divides by the squared norm",
     [("double y = nrm > 0.0 ? h[i] / nrm : 0.0;", "double y = nrm > 0.0 ? h[i] / ss : 0.0;", 0)]),
    ("mse decoder scales by 1/sqrt(d)",
     [("double scale = (double)norms[r] / d;", "double scale = (double)norms[r] / sqrt((double)d);", 0)]),
    ("mse decoder without D",
     [("store_elem(out, out_dtype, r * d + i, s[i] * z[i]);", "store_elem(out, out_dtype, r * d + i, z[i]);", 0)]),
    ("eden scale from the norm instead of its square",
     [("d * ss / ch", "d * nrm / ch", 0)]),
    ("biased drive scale over sqrt(d)",
     [("S = l1 / d;", "S = l1 / rd;", 0)]),
    ("drive decoder over d",
     [("S * s[i] * z[i] / rd);", "S * s[i] * z[i] / d);", 0)]),
    ("residual without its 1/sqrt(d)",
     [("ri = (h[i] - nrm * lv[code]) / rd;", "ri = (h[i] - nrm * lv[code]);", 0)]),
    ("residual decoder sign",
     [("(get_field(srow, i, 1) ? sr : -sr);", "(get_field(srow, i, 1) ? -sr : sr);", 0)]),
    ("score without the key factor",
     [("logits[(int64_t)j * n + k] = (float)(a * acc);", "logits[(int64_t)j * n + k] = (float)(acc);", 0)]),
    ("sign score over d",
     [("(float)((double)scale[k] / rd * acc);", "(float)((double)scale[k] / d * acc);", 0)]),
    ("residual score without 1/sqrt(d)",
     [("(double)res_scale[k] / rd * as);", "(double)res_scale[k] * as);", 0)]),
    ("attention without the logit scale",
     [("logit[j] = scale * acc;", "logit[j] = acc;", 0)]),
    ("rotated attention with the key signs on the values",
     [("for (t = 0; t < d; ++t) z[t] *= sv[t];", "for (t = 0; t < d; ++t) z[t] *= sk[t];", 0)]),
    ("rotated attention not normalized",
     [("for (t = 0; t < d; ++t) z[t] /= sum;", "for (t = 0; t < d; ++t) z[t] /= 1.0;", 0)]),
    ("fp16 subnormal exponent",
     [("v = ldexp((double)man, -24);", "v = ldexp((double)man, -25);", 0)]),
    ("fp16 normal exponent",
     [("v = ldexp((double)(man + 1024), exp - 25);", "v = ldexp((double)(man + 1024), exp - 24);", 0)]),
    ("fp16 overflow point",
     [("if (a >= 65520.0)", "if (a > 65504.0)", 0)]),
    ("lloyd-max centroid sign",
     [("double cn = (pa - pb) / std_prob(t[k], t[k + 1]);", "double cn = (pb - pa) / std_prob(t[k], t[k + 1]);", 0)]),
    ("finite-d density without the Jacobian",
     [("pow(cos(th), (double)(d - 2))", "pow(cos(th), (double)(d - 3))", 0)]),
    ("msb-first packing (writer and reader)",
     [("int64_t bit = (int64_t)w * i + j;", "int64_t bit = (int64_t)w * i + (w - 1 - j);", 0),
      ("int64_t bit = (int64_t)w * i + j;", "int64_t bit = (int64_t)w * i + (w - 1 - j);", 0)]),
]


def scratch_copy(dst):
    os.makedirs(os.path.join(dst, "oracle"))
    for f in ("__init__.py", "rht_oracle.c"):
        shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(dst, "oracle", f))
    os.makedirs(os.path.join(dst, "tests"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))


def replace_nth(text, old, new, k):
    at = -1
    for _ in range(k + 1):
        at = text.find(old, at + 1)
        if at < 0:
            return None
    return text[:at] + new + text[at + len(old):]


def run_pins(root):
    env = dict(os.environ, PYTHONPATH=root)
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
                           "-p", "no:cacheprovider"], cwd=root, env=env, capture_output=True, text=True)


def run_case(base, index, edits):
    """Pins on a copy with `edits` applied (none: the unchanged oracle).
    Returns (returncode, output), or None when an edit's text is not found."""
    root = os.path.join(base, "case%02d" % index)
    scratch_copy(root)
    src = os.path.join(root, "oracle", "rht_oracle.c")
    with open(src) as f:
        text = f.read()
    for old, new, k in edits:
        text = replace_nth(text, old, new, k)
        if text is None:
            return None
    with open(src, "w") as f:
        f.write(text)
    r = run_pins(root)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    base = str(tmp_path_factory.mktemp("mutations"))
    cases = [[]] + [edits for _, edits in MUTATIONS]
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(lambda ie: run_case(base, ie[0], ie[1]), enumerate(cases)))


def test_unchanged_copy_passes(outcomes):
    rc, out = outcomes[0]
    assert rc == 0, out


@pytest.mark.parametrize("index", range(len(MUTATIONS)), ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(outcomes, index):
    what = MUTATIONS[index][0]
    res = outcomes[index + 1]
    assert res is not None, "the rule to change is not in the oracle as expected: %s" % what
    rc, out = res
    assert rc != 0, "no pin fails when the oracle gets this wrong: %s" % what
    assert "failed" in out, out
