"""GPU parity at the edges of the input contract (include/rht.h: any finite
input whose ||x||^2 is a normal fp32 number or 0), on every encoder family the
workloads use: the d = 128 fp16 4-bit MFMA encoder and decoder, the d = 256
fp16 residual chain on MFMA, the generic butterfly kernels (d = 1024 fp16 and
fp32, d = 128 fp32) and DRIVE sign codes.

Rows: fp16 rows made entirely of subnormal numbers (including rows whose only
nonzero entry is the smallest subnormal, 2^-24), fp16 rows whose entries sit
near the largest finite value 65504 (and at it), and fp32 rows scaled by
1e17 and 1e-18 (||x||^2 stays a normal fp32 number).  Rules as everywhere
(tests/parity.py): codes bit-exact except near-threshold, norms and scales
relative 1e-6 / 1e-5, decodes of the GPU's codes within 1e-5 (fp32 out) of
the oracle's.  fp16 decodes of rows near 65504 can round past the largest
finite value, and decodes of the scaled fp32 rows fall outside fp16's range,
so those rows are decoded to fp32 only.
"""
import sys

import numpy as np
import pytest

import oracle
import rotation_vector_quantization_amd as rht
from parity import (NORM_RTOL, RECON_F16, RECON_F32, SCALE_RTOL, check_codes, check_recon, check_rel, unpack)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    rht.load()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def subnormal_f16_rows(n, d, rng):
    """fp16 rows whose every entry is subnormal (|x| < 2^-14), random signs and
    mantissas; row 0 holds only the smallest subnormal at one coordinate, row 1
    the smallest subnormal everywhere, row 2 the largest subnormal everywhere."""
    man = rng.integers(1, 1024, size=(n, d)).astype(np.uint16)
    sign = (rng.integers(0, 2, size=(n, d)).astype(np.uint16) << 15)
    x = (man | sign).view(np.float16)
    x[0] = 0.0
    x[0, d // 5] = np.uint16(1).view(np.float16)
    x[1] = np.uint16(1).view(np.float16)
    x[2] = np.uint16(1023).view(np.float16)
    assert np.all(np.abs(x.astype(np.float64)) < 2.0 ** -14)
    return x


def near_max_f16_rows(n, d, rng):
    """fp16 rows with entries of magnitude 30000 ... 65504, random signs; row 0
    is +-65504 everywhere, row 1 has one entry at 65504 and the rest small."""
    mag = rng.uniform(30000.0, 65504.0, size=(n, d))
    x = (mag * rng.choice([-1.0, 1.0], size=(n, d))).astype(np.float16)
    x[0] = 65504.0 * rng.choice([-1.0, 1.0], size=d)
    x[1] = rng.standard_normal(d)
    x[1, 3] = 65504.0
    assert np.all(np.isfinite(x))
    return x


def scaled_f32_rows(n, d, rng, scale):
    x = rng.standard_normal((n, d)) * scale
    x[:, 7] *= 20.0
    return x.astype(np.float32)


def check_mse(x, d, bits, seed, what, f16_decode=True):
    codes, norms = (host(t) for t in rht.quantize(dev(x), bits, seed))
    ocodes, onorms = oracle.quantize(x, bits, seed)
    _, th, _, _ = oracle.lloyd_max(bits)
    near = check_codes(unpack(codes, bits, d), unpack(ocodes, bits, d),
                       lambda rows: oracle.quantize(x[rows], bits, seed, want_y=True)[2], th, what + " codes")
    check_rel(norms, onorms, NORM_RTOL, what + " norms")
    outs = (("f32", torch.float32, np.float32, RECON_F32),) + (
        (("f16", torch.float16, np.float16, RECON_F16),) if f16_decode else ())
    for name, tdt, ndt, tol in outs:
        y = host(rht.dequantize(dev(codes), dev(norms), d, bits, seed, dtype=tdt))
        ref = oracle.dequantize(codes, norms, d, bits, seed, ndt)
        check_recon(y, ref, tol, "%s decode %s" % (what, name))
    say("%s: %d rows, %d near-threshold codes" % (what, x.shape[0], near))


def check_residual(x, d, bits, seed, what, f16_decode=True):
    codes, sg, norms, rs = (host(t) for t in rht.residual_quantize(dev(x), bits, seed))
    ocodes, _, onorms, _ = oracle.residual_quantize(x, bits, seed)
    _, th1, _, _ = oracle.lloyd_max(bits - 1)
    check_codes(unpack(codes, bits - 1, d), unpack(ocodes, bits - 1, d),
                lambda rows: oracle.quantize(x[rows], bits - 1, seed, want_y=True)[2], th1, what + " stage 1")
    check_rel(norms, onorms, NORM_RTOL, what + " norms")
    # sign bits and S_r on the GPU's own stage-1 codes
    _, fsg, _, frs = oracle.residual_quantize(x, bits, seed, forced_codes=codes)
    same = (sg == fsg).all(1)
    assert same.mean() > 0.99, what + ": residual sign bits differ on many rows"
    check_rel(rs[same], frs[same], SCALE_RTOL, what + " S_r")
    outs = (("f32", torch.float32, np.float32, RECON_F32),) + (
        (("f16", torch.float16, np.float16, RECON_F16),) if f16_decode else ())
    for name, tdt, ndt, tol in outs:
        y = host(rht.residual_dequantize(dev(codes), dev(sg), dev(norms), dev(rs), d, bits, seed, dtype=tdt))
        ref = oracle.residual_dequantize(codes, sg, norms, rs, d, bits, seed, ndt)
        check_recon(y, ref, tol, "%s decode %s" % (what, name))
    say("%s: %d rows" % (what, x.shape[0]))


def check_drive(x, d, seed, what):
    for unbiased, mode in ((False, rht.SCALE_SIGN_BIASED), (True, rht.SCALE_SIGN_UNBIASED)):
        b, S = (host(t) for t in rht.quantize(dev(x), 1, seed, mode))
        ob, oS = oracle.sign_quantize(x, unbiased, seed)
        check_codes(unpack(b, 1, d), unpack(ob, 1, d),
                    lambda rows: oracle.sign_quantize(x[rows], False, seed, want_y=True)[2],
                    np.array([0.0]), what + " bits")
        check_rel(S, oS, SCALE_RTOL, what + " S")
        y = host(rht.dequantize(dev(b), dev(S), d, 1, seed, mode, dtype=torch.float32))
        check_recon(y, oracle.sign_dequantize(b, S, d, seed, np.float32), RECON_F32, what + " decode")
    say("%s: %d rows" % (what, x.shape[0]))


# (d, bits) of the MSE encoders: the KV-block MFMA kernels (128, 4) and the
# generic ones
MSE_F16 = [(128, 4), (128, 2), (1024, 4), (256, 3), (16, 3), (16, 4)]


@pytest.mark.parametrize("d,bits", MSE_F16)
def test_mse_subnormal_f16_rows(d, bits):
    x = subnormal_f16_rows(333, d, np.random.default_rng(d + bits))
    check_mse(x, d, bits, 11 + d, "subnormal fp16 d=%d b=%d" % (d, bits))


@pytest.mark.parametrize("d,bits", MSE_F16)
def test_mse_near_max_f16_rows(d, bits):
    x = near_max_f16_rows(333, d, np.random.default_rng(7 * d + bits))
    check_mse(x, d, bits, 12 + d, "near-65504 fp16 d=%d b=%d" % (d, bits), f16_decode=False)


@pytest.mark.parametrize("scale", [1e17, 1e-18])
@pytest.mark.parametrize("d,bits", [(128, 4), (1024, 4), (256, 2), (16, 2)])
def test_mse_scaled_f32_rows(d, bits, scale):
    x = scaled_f32_rows(333, d, np.random.default_rng(d + int(np.log10(scale)) + 40), scale)
    assert np.all(np.isfinite((x.astype(np.float64) ** 2).sum(1).astype(np.float32)))
    # decoded values of 1e17-scaled rows are past fp16's range, of 1e-18-scaled rows below it
    check_mse(x, d, bits, 13 + d, "fp32 x %g d=%d b=%d" % (scale, d, bits), f16_decode=False)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [256, 16])
def test_residual_contract_edges(d, bits):
    rng = np.random.default_rng(90 + bits + d)
    check_residual(subnormal_f16_rows(250, d, rng), d, bits, 21, "residual subnormal fp16 d=%d b=%d" % (d, bits))
    check_residual(near_max_f16_rows(250, d, rng), d, bits, 22, "residual near-65504 fp16 d=%d b=%d" % (d, bits),
                   f16_decode=False)
    for scale in (1e17, 1e-18):
        check_residual(scaled_f32_rows(250, d, rng, scale), d, bits, 23,
                       "residual fp32 x %g d=%d b=%d" % (scale, d, bits), f16_decode=False)


@pytest.mark.parametrize("d", [16, 128, 1024])
def test_drive_contract_edges(d):
    rng = np.random.default_rng(300 + d)
    check_drive(subnormal_f16_rows(200, d, rng), d, 31, "drive subnormal fp16 d=%d" % d)
    check_drive(near_max_f16_rows(200, d, rng), d, 32, "drive near-65504 fp16 d=%d" % d)
    for scale in (1e17, 1e-18):
        check_drive(scaled_f32_rows(200, d, rng, scale), d, 33, "drive fp32 x %g d=%d" % (scale, d))
