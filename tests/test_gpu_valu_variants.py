"""The butterfly (register/DPP) versions of the kernels that run the Hadamard
transform on MFMA by default, selected with RHT_HADAMARD=valu, against the
oracle: the same parity grids, run in one child process that has the
variable set from its start (the library reads it once).  These variants
exist for the MFMA-against-butterflies comparison of the transform."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_valu_hadamard_variants_match_the_oracle():
    torch = pytest.importorskip("torch")
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    env = dict(os.environ, RHT_HADAMARD="valu")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "valu_variants_child.py")], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    print(r.stdout[-4000:], flush=True)
    assert r.returncode == 0, r.stdout[-4000:]
