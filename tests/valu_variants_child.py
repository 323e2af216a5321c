"""Child process of test_gpu_valu_variants.py: runs the parity checks whose
kernels RHT_HADAMARD=valu swaps for the register/DPP butterfly versions
(d = 128 fp16 4-bit MSE encode and decode, d = 256 fp16 residual chain,
d = 128 scoring of MSE, sign and residual codes).  The library reads the
variable once, at its first call, so it must be set before this process
starts.  Exits non-zero on the first failure.  Not collected by pytest."""
import os
import sys
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402

import rotation_vector_quantization_amd as rht  # noqa: E402
import test_gpu_parity as P  # noqa: E402
import test_gpu_scoring as S  # noqa: E402


def main():
    assert os.environ.get("RHT_HADAMARD") == "valu", "run with RHT_HADAMARD=valu"
    rht.load()
    cases = []
    for xdt in ("f16", "f32"):
        cases.append(("mse grid d=128 b=4 " + xdt, lambda xdt=xdt: P.test_mse_roundtrip_grid(128, 4, xdt)))
        cases.append(("finite-d grid d=128 b=4 " + xdt, lambda xdt=xdt: P.test_beta_codebook_grid(128, 4, xdt)))
    for bits in (2, 3, 4):
        cases.append(("residual grid d=256 b=%d" % bits, lambda b=bits: P.test_residual_grid(256, b, "f16")))
        cases.append(("residual extreme d=256 b=%d" % bits,
                      lambda b=bits: P.test_residual_extreme_rotated_coordinate(b, "f16")))
    for bits in (2, 3):
        for n in (1, 17, 1000):
            cases.append(("residual decode arbitrary b=%d n=%d" % (bits, n),
                          lambda b=bits, n=n: P.test_residual_decode_arbitrary_inputs(b, n)))
    shapes = [(1, 1), (17, 100), (64, 1037), (33, 31), (40, 65), (32, 64)]
    for bits in (1, 2, 3, 4):
        for m, n in shapes:
            cases.append(("score d=128 b=%d m=%d n=%d" % (bits, m, n),
                          lambda b=bits, m=m, n=n: P.test_score_grid(128, b, m, n)))
        if bits in (1, 4):
            cases.append(("score query scales b=%d" % bits, lambda b=bits: P.test_score_query_scales(b)))
    for unbiased in (False, True):
        for m, n in shapes:
            cases.append(("sign score d=128 unbiased=%d m=%d n=%d" % (unbiased, m, n),
                          lambda u=unbiased, m=m, n=n: S.test_sign_score_grid(u, 128, m, n)))
    for bits in (2, 3, 4):
        for m, n in shapes:
            cases.append(("residual score d=128 b=%d m=%d n=%d" % (bits, m, n),
                          lambda b=bits, m=m, n=n: S.test_residual_score_grid(b, 128, m, n)))
    for name, fn in cases:
        print("valu variant:", name, flush=True)
        try:
            fn()
        except Exception:
            traceback.print_exc()
            print("FAILED:", name, flush=True)
            return 1
    print("all %d valu-variant cases passed" % len(cases), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
