"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute: a value
printed on the web page "Random-rotation quantization" (fixtures under
``tests/golden`` with their citation), a closed form, a library routine
(scipy's Sylvester Hadamard matrix, numerical integration, numpy's fp16
conversion), an invariant, or brute force on tiny inputs.  Together they are
chosen so a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.special
import scipy.stats

import oracle


def _read_golden(path):
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            vals[k] = [float(t) for t in v]
    return vals


def unpack_fields(codes, width, d):
    """Independent LSB-first unpacker: field i of a row at bits [w*i, w*i+w)."""
    bits = np.unpackbits(codes, axis=-1, bitorder="little")[..., : width * d]
    bits = bits.reshape(*codes.shape[:-1], d, width).astype(np.int64)
    return (bits << np.arange(width)).sum(-1)


def dense_rotation(d, seed):
    """H D as a dense matrix, H from scipy (Sylvester order), D from the oracle."""
    return scipy.linalg.hadamard(d).astype(np.float64) * oracle.signs(seed, d)[None, :].astype(np.float64)


# ---------------------------------------------------------------- generator
def test_splitmix64_known_answer():
    # Published first outputs of SplitMix64 started from state 0.
    assert oracle.splitmix64_stream(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                             0x06C45D188009454F]
    # sign i is the top bit of output i (set -> -1)
    assert list(oracle.signs(0, 3)) == [-1, 1, 1]


def test_signs_deterministic_and_balanced():
    a = oracle.signs(42, 4096)
    assert np.array_equal(a, oracle.signs(42, 4096))
    assert not np.array_equal(a, oracle.signs(43, 4096))
    assert set(np.unique(a)) <= {-1, 1}
    frac = np.mean([(oracle.signs(s, 1024) > 0).mean() for s in range(64)])
    assert abs(frac - 0.5) < 0.01
    # prefix property: the first d signs do not depend on d
    assert np.array_equal(oracle.signs(7, 128), oracle.signs(7, 1024)[:128])


# ---------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64])
def test_fwht_matches_dense_sylvester(d):
    rng = np.random.default_rng(d)
    v = rng.standard_normal((5, d))
    H = scipy.linalg.hadamard(d).astype(np.float64)
    np.testing.assert_allclose(oracle.fwht(v), v @ H.T, rtol=0, atol=1e-12)


def test_fwht_d2_and_orthogonality():
    np.testing.assert_array_equal(oracle.fwht(np.eye(2)), [[1, 1], [1, -1]])
    for d in (8, 64, 256):
        H = oracle.fwht(np.eye(d))
        np.testing.assert_array_equal(H @ H.T, d * np.eye(d))          # H H^T = d I exactly
        P = H / math.sqrt(d)
        np.testing.assert_allclose(P @ P, np.eye(d), atol=1e-12)        # (H/sqrt d)^2 = I


@pytest.mark.parametrize("d", [16, 128, 1024, 4096])
def test_rotation_preserves_norm(d):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((8, d)).astype(np.float32)
    _, norms, y = oracle.quantize(x, 4, 11, want_y=True)
    nx = np.linalg.norm(x.astype(np.float64), axis=1)
    # y = H D x / ||x||, so ||y|| = sqrt(d) exactly when Pi is orthogonal
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), math.sqrt(d), rtol=1e-12)
    np.testing.assert_allclose(norms, nx.astype(np.float32), rtol=0)


# ---------------------------------------------------------- rotated marginal
def test_rotated_coordinate_mean_and_std(golden_dir):
    """[RRQ 'Why rotation works']: mean 0, std 1/sqrt(d) per coordinate."""
    g = _read_golden(golden_dir + "/rrq_rotation_stats.txt")
    d, trials = 64, 4000
    x = np.zeros((1, d), np.float32)
    x[0, 5] = 0.6
    x[0, 40] = 0.8  # unit vector with its energy in two channels
    xs = np.repeat(x, 1, axis=0)
    vals = np.stack([oracle.quantize(xs, 1, s, want_y=True)[2][0] / math.sqrt(d) for s in range(trials)])
    # over seeds, every coordinate of Pi x has mean 0 and variance ||x||^2 / d
    assert abs(vals.mean()) < 4.0 / math.sqrt(trials * d) * 1.0
    np.testing.assert_allclose(vals.var(axis=0).mean(), 1.0 / d, rtol=0.03)
    # page value: std ~0.032 at d ~ 1000; at d = 1024 the exact value is 1/32
    d2 = 1024
    rng = np.random.default_rng(3)
    x2 = rng.standard_normal((64, d2)).astype(np.float32)
    y2 = oracle.quantize(x2, 1, 5, want_y=True)[2] / math.sqrt(d2)
    assert abs(y2.std() - g["std"][0]) < 0.0015
    assert abs(y2.mean() - g["mean"][0]) < 0.002


def _beta_marginal_pdf(x, d):
    # the page's density of one coordinate on the unit sphere (garbled
    # "\sqrt{\pi},\Gamma" read as sqrt(pi) * Gamma)
    c = math.exp(math.lgamma(d / 2) - math.lgamma((d - 1) / 2)) / math.sqrt(math.pi)
    return c * (1.0 - x * x) ** ((d - 3) / 2)


@pytest.mark.parametrize("d", [8, 16, 128])
def test_beta_marginal_ks(d):
    """Gaussian inputs rotate to a uniform point on the sphere exactly, so one
    coordinate of Pi x / ||x|| follows the page's Beta marginal."""
    total, _ = scipy.integrate.quad(_beta_marginal_pdf, -1, 1, args=(d,))
    assert abs(total - 1.0) < 1e-9
    rng = np.random.default_rng(d)
    x = rng.standard_normal((3000, d)).astype(np.float64).astype(np.float32)
    y = oracle.quantize(x, 2, 99, want_y=True)[2]
    sample = y[:, d // 3] / math.sqrt(d)

    def cdf(t):
        t = np.atleast_1d(t)
        return np.array([scipy.integrate.quad(_beta_marginal_pdf, -1, min(max(v, -1), 1), args=(d,))[0]
                         for v in t])

    p = scipy.stats.kstest(sample, cdf).pvalue
    assert p > 1e-3


# ---------------------------------------------------------------- codebook
def test_lloyd_max_page_values(golden_dir):
    g = _read_golden(golden_dir + "/rrq_codebook.txt")
    lv1, th1, mse1, _ = oracle.lloyd_max(1)
    assert abs(lv1[1] - g["sqrt_2_over_pi_1bit"][0]) < 1e-3
    np.testing.assert_allclose(lv1, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-13)
    assert th1[0] == 0.0
    assert abs(mse1 - (1 - 2 / math.pi)) < 1e-13      # 1-bit Gaussian MSE, closed form
    lv2, th2, _, _ = oracle.lloyd_max(2)
    np.testing.assert_allclose(lv2[2:], g["levels_2bit_positive"], atol=1e-3)
    np.testing.assert_allclose(lv2[:2], -lv2[2:][::-1], atol=0)


def test_lloyd_max_textbook_table(golden_dir):
    g = _read_golden(golden_dir + "/max1960_lloyd_max.txt")
    for b in (3, 4):
        lv, th, mse, _ = oracle.lloyd_max(b)
        np.testing.assert_allclose(lv[1 << (b - 1):], g["levels_%dbit_positive" % b], atol=1.1e-3)
        assert abs(mse - g["mse_%dbit" % b][0]) < 1e-5


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_lloyd_max_fixed_point_by_quadrature(b):
    """Centroid and nearest-neighbour conditions, checked by numerical
    integration rather than the oracle's closed-form cell means."""
    lv, th, mse, _ = oracle.lloyd_max(b)
    K = 1 << b
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    phi = scipy.stats.norm.pdf
    dist = 0.0
    for k in range(K):
        a, c = edges[k], edges[k + 1]
        p, _ = scipy.integrate.quad(phi, a, c)
        m1, _ = scipy.integrate.quad(lambda z: z * phi(z), a, c)
        assert abs(m1 / p - lv[k]) < 1e-9
        e, _ = scipy.integrate.quad(lambda z: (z - lv[k]) ** 2 * phi(z), a, c)
        dist += e
    np.testing.assert_allclose(th, 0.5 * (lv[1:] + lv[:-1]), atol=1e-15)
    assert abs(dist - mse) < 1e-9
    assert np.all(np.diff(lv) > 0)


def test_one_bit_mse_monte_carlo():
    z = np.random.default_rng(7).standard_normal(2_000_000)
    e = np.mean((z - math.sqrt(2 / math.pi) * np.sign(z)) ** 2)
    assert abs(e - (1 - 2 / math.pi)) < 2e-3


# ---------------------------------------------------------------- encoder
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [8, 16, 32])
@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_quantize_bruteforce(bits, d, dt):
    rng = np.random.default_rng(bits * 100 + d)
    x = (rng.standard_normal((40, d)) * 3).astype(dt)
    seed = 1234 + d
    codes, norms = oracle.quantize(x, bits, seed)
    lv, _, _, _ = oracle.lloyd_max(bits)
    xd = x.astype(np.float64)
    nx = np.linalg.norm(xd, axis=1)
    y = xd @ dense_rotation(d, seed).T / nx[:, None]
    brute = np.argmin(np.abs(y[..., None] - lv[None, None, :]), axis=-1)
    got = unpack_fields(codes, bits, d)
    np.testing.assert_array_equal(got, brute)
    np.testing.assert_array_equal(norms, nx.astype(np.float32))


def test_quantize_zero_vector_and_ties():
    d = 16
    x = np.zeros((2, d), np.float32)
    for bits in (1, 2, 4):
        codes, norms = oracle.quantize(x, bits, 3)
        assert np.all(unpack_fields(codes, bits, d) == (1 << bits) // 2)
        assert np.all(norms == 0)
        out = oracle.dequantize(codes, norms, d, bits, 3)
        assert np.all(out == 0)
    # a vector whose rotation has exact zeros: y = 0 goes up to code K/2
    x = np.zeros((1, d), np.float32)
    s = oracle.signs(3, d)
    x[0, 0] = s[0]
    x[0, 1] = s[1]          # H D x = H (e0 + e1): half the coordinates are 0
    codes, _ = oracle.quantize(x, 2, 3)
    c = unpack_fields(codes, 2, d)[0]
    y = oracle.fwht(np.array([[1.0, 1.0] + [0.0] * (d - 2)]))[0]
    assert np.all(c[y == 0] == 2)


def test_fp16_codec_against_numpy():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    ours = np.array([oracle.f16_to_f64(int(b)) for b in allbits])
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(ours[finite], ref[finite])
    assert np.all(np.isnan(ours[np.isnan(ref)]))
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(3000) * s for s in (1e-7, 1e-5, 1, 100, 3e4)]
                       + [np.array([65504.0, 65519.99, 65520.0, 2.0 ** -25, 2.0 ** -24 * 1.5, -0.0])])
    ours = np.array([oracle.f64_to_f16(float(t)) for t in v], dtype=np.uint16)
    with np.errstate(over="ignore"):  # values past 65520 round to infinity on purpose
        want = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, want)


def test_fp16_encoder_rounds_exact_ties_to_even():
    """Values exactly halfway between two fp16 numbers, (2k+1) 2^(e-11) for a
    in [2^e, 2^(e+1)), over the whole normal range and in the subnormal range
    ((2k+1) 2^-25): round-to-nearest-even picks the neighbour with an even
    significand, which numpy's conversion fixes independently."""
    ties = []
    for e in (-14, -13, -7, -1, 0, 1, 4, 10, 14, 15):
        k = np.arange(1024, 2048, dtype=np.float64)       # significand m, a = (m + 1/2) 2^(e-10)
        ties.append((2 * k + 1) * 2.0 ** (e - 11))
    ties.append((2 * np.arange(0, 1024, dtype=np.float64) + 1) * 2.0 ** -25)
    v = np.concatenate(ties)
    v = v[v < 65520.0]                                    # 65520 itself rounds to infinity
    v = np.concatenate([v, -v])
    ours = np.array([oracle.f64_to_f16(float(t)) for t in v], dtype=np.uint16)
    want = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, want)
    # each tie went to the even significand, not away from zero
    assert np.all((ours & 1) == 0)
    up = np.abs(v) < np.abs(ours.view(np.float16).astype(np.float64))
    assert 0 < up.mean() < 1                              # both directions occur


# ---------------------------------------------------------------- decoders
@pytest.mark.parametrize("bits", [1, 2, 4])
def test_dequantize_dense_and_rotated_domain_error(bits):
    d, seed = 64, 77
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((20, d)).astype(np.float32)
    codes, norms = oracle.quantize(x, bits, seed)
    lv, _, _, _ = oracle.lloyd_max(bits)
    c = lv[unpack_fields(codes, bits, d)]
    R = dense_rotation(d, seed)                      # H D
    xt = (c * (norms.astype(np.float64)[:, None] / d)) @ R   # D H z = (H D)^T z
    got = oracle.dequantize(codes, norms, d, bits, seed).astype(np.float64)
    np.testing.assert_allclose(got, xt, rtol=0, atol=1e-6 * np.abs(xt).max())
    # ||x - x~|| in the original domain equals ||Pi x - y^|| in the rotated one
    xd = x.astype(np.float64)
    Pi = R / math.sqrt(d)
    yhat = c * norms.astype(np.float64)[:, None] / math.sqrt(d)
    np.testing.assert_allclose(np.linalg.norm(xd - xt, axis=1),
                               np.linalg.norm(xd @ Pi.T - yhat, axis=1), rtol=1e-9)
    f16 = oracle.dequantize(codes, norms, d, bits, seed, np.float16)
    np.testing.assert_array_equal(f16, xt.astype(np.float16))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_distortion_matches_lloyd_max(bits):
    """For Gaussian inputs Pi x / ||x|| is uniform on the sphere and the
    normalized MSE approaches D_b (d large)."""
    d = 1024
    x = np.random.default_rng(bits).standard_normal((200, d)).astype(np.float32)
    codes, norms = oracle.quantize(x, bits, 5)
    xt = oracle.dequantize(codes, norms, d, bits, 5).astype(np.float64)
    xd = x.astype(np.float64)
    nmse = np.mean(np.sum((xd - xt) ** 2, 1) / np.sum(xd ** 2, 1))
    _, _, mse, _ = oracle.lloyd_max(bits)
    assert abs(nmse / mse - 1) < 0.03


@pytest.mark.parametrize("unbiased", [False, True])
def test_drive_closed_forms(unbiased):
    d, seed = 256, 21
    rng = np.random.default_rng(4)
    x = (rng.standard_t(3, size=(30, d))).astype(np.float32)
    b, S = oracle.sign_quantize(x, unbiased, seed)
    xd = x.astype(np.float64)
    Pi = dense_rotation(d, seed) / math.sqrt(d)
    Rx = xd @ Pi.T
    np.testing.assert_array_equal(unpack_fields(b, 1, d), (Rx >= 0).astype(np.int64))
    l1 = np.abs(Rx).sum(1)
    S_ref = (xd ** 2).sum(1) / l1 if unbiased else l1 / d
    np.testing.assert_allclose(S, S_ref.astype(np.float32), rtol=1e-6)
    xh = oracle.sign_dequantize(b, S, d, seed).astype(np.float64)
    S64 = S.astype(np.float64)
    sigma = np.where(Rx >= 0, 1.0, -1.0)
    np.testing.assert_allclose(xh, (S64[:, None] * sigma) @ Pi, rtol=0, atol=1e-6 * np.abs(xh).max())
    if unbiased:
        # <x, x^> = S ||Rx||_1 = ||x||^2
        np.testing.assert_allclose((xd * xh).sum(1), (xd ** 2).sum(1), rtol=2e-6)
    else:
        # ||x - x^||^2 = ||x||^2 - ||Rx||_1^2 / d
        np.testing.assert_allclose(((xd - xh) ** 2).sum(1), (xd ** 2).sum(1) - l1 ** 2 / d, rtol=2e-5)


def test_drive_unbiased_mean_over_seeds():
    d, trials = 32, 3000
    x = np.random.default_rng(9).standard_normal((1, d)).astype(np.float32)
    acc = np.zeros(d)
    for s in range(trials):
        b, S = oracle.sign_quantize(x, True, 1000 + s)
        acc += oracle.sign_dequantize(b, S, d, 1000 + s)[0]
    err = np.linalg.norm(acc / trials - x[0]) / np.linalg.norm(x[0])
    assert err < 4.0 / math.sqrt(trials) * math.sqrt(d) / 4


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_residual_chain_closed_forms(bits):
    d, seed = 128, 31
    rng = np.random.default_rng(bits + 50)
    x = rng.standard_normal((25, d)).astype(np.float32)
    x[:, 7] *= 30
    codes, sg, norms, rs = oracle.residual_quantize(x, bits, seed)
    c1, n1 = oracle.quantize(x, bits - 1, seed)
    np.testing.assert_array_equal(codes, c1)          # stage 1 = (b-1)-bit encoder
    np.testing.assert_array_equal(norms, n1)
    lv, _, _, _ = oracle.lloyd_max(bits - 1)
    xd = x.astype(np.float64)
    R = dense_rotation(d, seed)
    nx = np.linalg.norm(xd, axis=1)
    cz = lv[unpack_fields(codes, bits - 1, d)]
    r = (xd @ R.T - nx[:, None] * cz) / math.sqrt(d)    # Pi (x - x~)
    np.testing.assert_array_equal(unpack_fields(sg, 1, d), (r >= 0).astype(np.int64))
    Sr = (r ** 2).sum(1) / np.abs(r).sum(1)
    np.testing.assert_allclose(rs, Sr.astype(np.float32), rtol=1e-6)
    xh = oracle.residual_dequantize(codes, sg, norms, rs, d, bits, seed).astype(np.float64)
    r2, r1 = (r ** 2).sum(1), np.abs(r).sum(1)
    np.testing.assert_allclose(((xd - xh) ** 2).sum(1), r2 * (d * r2 / r1 ** 2 - 1), rtol=1e-4)
    # forcing the stage-1 codes to the oracle's own gives identical results
    f = oracle.residual_quantize(x, bits, seed, forced_codes=codes)
    for a, b in zip(f, (codes, sg, norms, rs)):
        np.testing.assert_array_equal(a, b)


# ------------------------------------------- edge readings of the sign codes
# The pages give no rule for a rotated coordinate that is exactly 0 or for a
# zero vector.  The readings: a sign bit is [v >= 0], so +0 and -0 both give
# bit 1 (the 1-bit code then equals the 1-bit Lloyd-Max code index, whose
# middle threshold 0 goes up); a scale whose definition is 0/0 is 0, so a
# zero vector decodes to exactly 0.  Each value below is fixed by that
# reading, computed here by hand, not by the oracle.
def _exact_zero_rows(d, seed):
    """x = s_0 e_0 + s_1 e_1 with s the rotation signs: D x = e_0 + e_1 and
    (H D x)_i = 1 + (-1)^i, so every odd rotated coordinate is exactly 0 and
    every even one is exactly 2.  Also its negation (odd coordinates -0 after
    the sign flips) and a zero row (its rotation holds both +0 and -0)."""
    s = oracle.signs(seed, d).astype(np.float32)
    x = np.zeros((3, d), np.float32)
    x[0, 0], x[0, 1] = s[0], s[1]
    x[1] = -x[0]
    return x


@pytest.mark.parametrize("dt", [np.float32, np.float16])
@pytest.mark.parametrize("unbiased", [False, True])
def test_drive_sign_bit_at_exact_zero_and_zero_vector(unbiased, dt):
    d, seed = 64, 19
    x = _exact_zero_rows(d, seed).astype(dt)
    b, S = oracle.sign_quantize(x, unbiased, seed)
    bits = unpack_fields(b, 1, d)
    odd = np.arange(d) % 2 == 1
    # row 0: H D x = 2 on even, +0 on odd -> every bit 1
    np.testing.assert_array_equal(bits[0], np.ones(d, np.int64))
    # row 1: -2 on even (bit 0), exact zero on odd (bit 1)
    np.testing.assert_array_equal(bits[1], odd.astype(np.int64))
    # row 2: the zero vector -> every bit 1, S = 0 in both modes
    np.testing.assert_array_equal(bits[2], np.ones(d, np.int64))
    # ||Pi x||_1 = (d/2) 2 / sqrt(d) = sqrt(d); ||x||^2 = 2
    want = 2.0 / math.sqrt(d) if unbiased else math.sqrt(d) / d
    np.testing.assert_allclose(S[:2], [want, want], rtol=1e-7)
    assert S[2] == 0.0 and not np.signbit(S[2])
    xh = oracle.sign_dequantize(b, S, d, seed)
    assert np.all(xh[2] == 0.0)
    # <x, x^> = S <Pi x, sigma> = S ||Pi x||_1: ||x||^2 = 2 (unbiased), ||Pi x||_1^2 / d = 1 (biased)
    np.testing.assert_allclose(float((x[0].astype(np.float64) * xh[0].astype(np.float64)).sum()),
                               2.0 if unbiased else 1.0, rtol=1e-6)


@pytest.mark.parametrize("dt", [np.float32, np.float16])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_residual_sign_bit_and_scale_at_zero(bits, dt):
    d, seed = 64, 23
    x = _exact_zero_rows(d, seed).astype(dt)
    codes, sg, norms, rs = oracle.residual_quantize(x, bits, seed)
    K1 = 1 << (bits - 1)
    # zero vector: stage-1 codes K1/2, norm 0, residual +-0 everywhere -> every
    # sign bit 1, S_r = 0/0 = 0, and the decode is exactly 0
    assert np.all(unpack_fields(codes[2:], bits - 1, d) == K1 // 2)
    assert norms[2] == 0.0 and rs[2] == 0.0 and not np.signbit(rs[2])
    np.testing.assert_array_equal(unpack_fields(sg[2:], 1, d)[0], np.ones(d, np.int64))
    y = oracle.residual_dequantize(codes, sg, norms, rs, d, bits, seed)
    assert np.all(y[2] == 0.0)
    # row 0: y = sqrt(2) on even coordinates, exact 0 on odd ones; the odd
    # coordinates take the first level above 0 and their residual is negative
    lv, _, _, _ = oracle.lloyd_max(bits - 1)
    c = unpack_fields(codes[:1], bits - 1, d)[0]
    assert np.all(c[1::2] == K1 // 2)
    sb = unpack_fields(sg[:1], 1, d)[0]
    assert np.all(sb[1::2] == 0)
    yev = math.sqrt(2.0)
    assert np.all(sb[0::2] == (1 if yev >= lv[c[0]] else 0))


def test_quantize_and_eden_zero_vector_scales():
    """MSE and EDEN codes of a zero vector: code K/2 everywhere, scale 0 (EDEN's
    d ||x||^2 / <c, H D x> is 0/0), decode exactly 0."""
    d = 32
    x = np.zeros((2, d), np.float16)
    for bits in (1, 2, 3, 4):
        c, S = oracle.quantize_eden(x, bits, 7)
        assert np.all(unpack_fields(c, bits, d) == (1 << bits) // 2)
        assert np.all(S == 0.0)
        assert np.all(oracle.dequantize(c, S, d, bits, 7, np.float16).astype(np.float64) == 0.0)


def test_residual_chain_removes_inner_product_shrinkage():
    """[RRQ 'Bias vs unbiasedness']: MSE codes shrink inner products by about
    1 - D_b; the residual chain is close to unbiased (diagnostic, loose)."""
    d, n = 256, 400
    rng = np.random.default_rng(5)
    x = rng.standard_normal((n, d)).astype(np.float32)
    q = rng.standard_normal((n, d))
    xd = x.astype(np.float64)
    true = (q * xd).sum(1)
    ratios_mse, ratios_res = [], []
    for s in range(6):
        c, nr = oracle.quantize(x, 2, 300 + s)
        xt = oracle.dequantize(c, nr, d, 2, 300 + s).astype(np.float64)
        ratios_mse.append(((q * xt).sum(1) * true).sum() / (true ** 2).sum())
        c3, s3, n3, r3 = oracle.residual_quantize(x, 3, 300 + s)
        xh = oracle.residual_dequantize(c3, s3, n3, r3, d, 3, 300 + s).astype(np.float64)
        ratios_res.append(((q * xh).sum(1) * true).sum() / (true ** 2).sum())
    _, _, D2, _ = oracle.lloyd_max(2)
    assert abs(np.mean(ratios_mse) - (1 - D2)) < 0.03
    assert abs(np.mean(ratios_res) - 1.0) < abs(np.mean(ratios_mse) - 1.0)


def test_score_equals_dense_definition():
    d, bits, seed = 128, 4, 46
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((50, d)).astype(np.float32)
    q = rng.standard_normal((7, d)).astype(np.float32)
    codes, norms = oracle.quantize(keys, bits, seed)
    dense = oracle.score_dense(q, codes, norms, d, bits, seed)
    lv, _, _, _ = oracle.lloyd_max(bits)
    xt = (lv[unpack_fields(codes, bits, d)] * norms.astype(np.float64)[:, None] / d) @ dense_rotation(d, seed)
    np.testing.assert_allclose(dense, q.astype(np.float64) @ xt.T, rtol=0, atol=1e-12 * np.abs(dense).max())
    fast = oracle.score(q, codes, norms, d, bits, seed)
    np.testing.assert_allclose(fast, dense, rtol=2e-7, atol=1e-9 * np.abs(dense).max())


# ---------------------------------------------------------------- attention
def _coded_heads(rng, heads, n, d, bits, seed, scale_rows=None):
    x = rng.standard_normal((heads * n, d)).astype(np.float32)
    if scale_rows is not None:
        x *= scale_rows
    c, nr = oracle.quantize(x, bits, seed)
    return c.reshape(heads, n, -1), nr.reshape(heads, n)


def _dense_decode(codes, norms, d, bits, seed):
    """Independent decoder: levels from the pinned codebook, an explicit dense
    Pi^T = (H D)^T / sqrt(d) from scipy, fields unpacked with numpy."""
    lv = oracle.lloyd_max(bits)[0]
    y = lv[unpack_fields(codes, bits, d)] / math.sqrt(d)
    return (y * norms[..., None].astype(np.float64)) @ (dense_rotation(d, seed) / math.sqrt(d))


@pytest.mark.parametrize("kbits,vbits,d", [(4, 4, 128), (2, 2, 64), (3, 3, 32), (1, 1, 16), (4, 3, 128),
                                           (3, 4, 64), (4, 2, 32), (2, 3, 128)])
def test_attention_matches_library_softmax_on_dense_decodes(kbits, vbits, d):
    # scipy's softmax over logits against an independently decoded K, V (each
    # with the codebook of its own width: 4-bit keys with 3-bit values is the
    # KV-cache pairing of "Practical use in llama.cpp")
    rng = np.random.default_rng(kbits * 100 + vbits * 10 + d)
    heads, m, n = 3, 4, 37
    kc, kn = _coded_heads(rng, heads, n, d, kbits, 7)
    vc, vn = _coded_heads(rng, heads, n, d, vbits, 9)
    q = rng.standard_normal((heads, m, d)).astype(np.float32)
    scale = 1.0 / math.sqrt(d)
    got = oracle.attention(q, kc, kn, vc, vn, d, kbits, vbits, 7, 9, scale)
    for b in range(heads):
        kd = _dense_decode(kc[b], kn[b], d, kbits, 7)
        vd = _dense_decode(vc[b], vn[b], d, vbits, 9)
        p = scipy.special.softmax(scale * (q[b].astype(np.float64) @ kd.T), axis=1)
        np.testing.assert_allclose(got[b], p @ vd, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("kbits,vbits", [(1, 1), (2, 2), (3, 3), (4, 4), (4, 3), (2, 4), (3, 1)])
@pytest.mark.parametrize("d", [32, 128, 256])
def test_attention_rotated_domain_equals_definition(kbits, vbits, d):
    # logits on the codes, value sum kept rotated, one inverse transform per query
    rng = np.random.default_rng(kbits + 8 * vbits + d)
    heads, m, n = 2, 5, 61
    kc, kn = _coded_heads(rng, heads, n, d, kbits, 21)
    vc, vn = _coded_heads(rng, heads, n, d, vbits, 22)
    q = (3 * rng.standard_normal((heads, m, d))).astype(np.float32)
    a = oracle.attention(q, kc, kn, vc, vn, d, kbits, vbits, 21, 22, 0.2)
    r = oracle.attention_rotated(q, kc, kn, vc, vn, d, kbits, vbits, 21, 22, 0.2)
    np.testing.assert_allclose(r, a, rtol=1e-12, atol=1e-12 * np.abs(a).max())


def test_attention_single_key_is_its_value():
    rng = np.random.default_rng(5)
    d, bits = 64, 4
    kc, kn = _coded_heads(rng, 2, 1, d, bits, 3)
    vc, vn = _coded_heads(rng, 2, 1, d, bits, 4)
    q = rng.standard_normal((2, 3, d)).astype(np.float32)
    got = oracle.attention_rotated(q, kc, kn, vc, vn, d, bits, bits, 3, 4, 0.5)
    for b in range(2):
        want = _dense_decode(vc[b], vn[b], d, bits, 4)[0]
        np.testing.assert_allclose(got[b], np.broadcast_to(want, (3, d)), rtol=1e-12, atol=1e-13)


def test_attention_uniform_weights_give_the_mean_value():
    # q = 0 (or scale = 0): every logit is equal, the output is the mean decode
    rng = np.random.default_rng(6)
    d, bits, n = 128, 2, 40
    kc, kn = _coded_heads(rng, 1, n, d, bits, 13)
    vc, vn = _coded_heads(rng, 1, n, d, bits, 14)
    want = _dense_decode(vc[0], vn[0], d, bits, 14).mean(0)
    q0 = np.zeros((1, 2, d), np.float32)
    q1 = rng.standard_normal((1, 2, d)).astype(np.float32)
    for q, s in ((q0, 1.0), (q1, 0.0)):
        got = oracle.attention_rotated(q, kc, kn, vc, vn, d, bits, bits, 13, 14, s)
        np.testing.assert_allclose(got[0], np.broadcast_to(want, (2, d)), rtol=1e-12, atol=1e-13)


def test_attention_large_scale_selects_the_best_key():
    rng = np.random.default_rng(8)
    d, bits, vbits, n = 64, 4, 3, 25
    kc, kn = _coded_heads(rng, 1, n, d, bits, 31)
    vc, vn = _coded_heads(rng, 1, n, d, vbits, 32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    kd = _dense_decode(kc[0], kn[0], d, bits, 31)
    logits = kd @ q[0, 0].astype(np.float64)
    best = int(np.argmax(logits))
    gap = np.sort(logits)[-1] - np.sort(logits)[-2]
    got = oracle.attention_rotated(q, kc, kn, vc, vn, d, bits, vbits, 31, 32, 60.0 / gap)
    want = _dense_decode(vc[0], vn[0], d, vbits, 32)[best]
    np.testing.assert_allclose(got[0, 0], want, rtol=1e-9, atol=1e-9 * np.abs(want).max())


def test_attention_key_permutation_and_value_scaling():
    rng = np.random.default_rng(9)
    d, bits, n = 32, 3, 30
    kc, kn = _coded_heads(rng, 1, n, d, bits, 41)
    vc, vn = _coded_heads(rng, 1, n, d, bits, 42)
    q = rng.standard_normal((1, 3, d)).astype(np.float32)
    base = oracle.attention_rotated(q, kc, kn, vc, vn, d, bits, bits, 41, 42, 0.3)
    perm = rng.permutation(n)
    got = oracle.attention_rotated(q, kc[:, perm], kn[:, perm], vc[:, perm], vn[:, perm], d, bits, bits,
                                   41, 42, 0.3)
    np.testing.assert_allclose(got, base, rtol=1e-12, atol=1e-14)
    # values enter linearly: doubling every value norm doubles the output
    got2 = oracle.attention_rotated(q, kc, kn, vc, 2 * vn, d, bits, bits, 41, 42, 0.3)
    np.testing.assert_allclose(got2, 2 * base, rtol=1e-12, atol=1e-14)
    # swapping the key and value seeds changes the result
    other = oracle.attention_rotated(q, kc, kn, vc, vn, d, bits, bits, 42, 41, 0.3)
    assert np.abs(other - base).max() > 1e-3 * np.abs(base).max()


# ------------------------------------------------- sign and residual scoring
@pytest.mark.parametrize("d", [8, 64, 256])
@pytest.mark.parametrize("unbiased", [False, True])
def test_sign_score_equals_definition_and_decoder(d, unbiased):
    rng = np.random.default_rng(d + unbiased)
    x = rng.standard_normal((50, d)).astype(np.float32)
    q = rng.standard_normal((7, d)).astype(np.float32)
    b, S = oracle.sign_quantize(x, unbiased, 17)
    rot = oracle.score_sign(q, b, S, d, 17).astype(np.float64)
    dense = oracle.score_sign(q, b, S, d, 17, dense=True)
    np.testing.assert_allclose(rot, dense, rtol=2e-7, atol=2e-7 * np.abs(dense).max())
    # the dense definition against the (separately pinned) mean decoder
    xh = oracle.sign_dequantize(b, S, d, 17).astype(np.float64)
    np.testing.assert_allclose(dense, q.astype(np.float64) @ xh.T, rtol=1e-6, atol=1e-6 * np.abs(dense).max())


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [16, 128])
def test_residual_score_equals_definition_and_decoder(bits, d):
    rng = np.random.default_rng(bits * d)
    x = rng.standard_normal((40, d)).astype(np.float32)
    q = rng.standard_normal((5, d)).astype(np.float32)
    c, g, nr, rs = oracle.residual_quantize(x, bits, 23)
    rot = oracle.score_residual(q, c, g, nr, rs, d, bits, 23).astype(np.float64)
    dense = oracle.score_residual(q, c, g, nr, rs, d, bits, 23, dense=True)
    np.testing.assert_allclose(rot, dense, rtol=2e-7, atol=2e-7 * np.abs(dense).max())
    xh = oracle.residual_dequantize(c, g, nr, rs, d, bits, 23).astype(np.float64)
    np.testing.assert_allclose(dense, q.astype(np.float64) @ xh.T, rtol=1e-6, atol=1e-6 * np.abs(dense).max())


def test_inner_product_bias_harness():
    # Monte Carlo over rotation seeds ("Bias vs unbiasedness"; "Three decoders"):
    # DRIVE's unbiased scale gives mean <q, x^> = <q, x>; the biased scale and
    # the MSE codes shrink it, the MSE codes by about 1 - D_b (centroid rule);
    # the residual chain (reading: same rotation, S_r = ||r||^2 / ||r||_1)
    # shrinks less than its own stage-1 code.
    rng = np.random.default_rng(1)
    d, seeds = 64, range(1500)
    x = rng.standard_normal((1, d)).astype(np.float32)
    q = (x + 0.5 * rng.standard_normal((1, d))).astype(np.float32)
    true = float(x[0].astype(np.float64) @ q[0].astype(np.float64))
    est = {k: [] for k in ("unb", "bia", "mse1", "mse2", "res2", "res3")}
    for s in seeds:
        b, S = oracle.sign_quantize(x, True, s)
        est["unb"].append(oracle.score_sign(q, b, S, d, s)[0, 0])
        b, S = oracle.sign_quantize(x, False, s)
        est["bia"].append(oracle.score_sign(q, b, S, d, s)[0, 0])
        for bb in (1, 2):
            c, nr = oracle.quantize(x, bb, s)
            est["mse%d" % bb].append(oracle.score(q, c, nr, d, bb, s)[0, 0])
        for bb in (2, 3):
            c, g, nr, rs = oracle.residual_quantize(x, bb, s)
            est["res%d" % bb].append(oracle.score_residual(q, c, g, nr, rs, d, bb, s)[0, 0])
    r = {k: np.mean(v) / true for k, v in est.items()}
    se = {k: np.std(v) / np.sqrt(len(v)) / true for k, v in est.items()}
    assert abs(r["unb"] - 1) < 5 * se["unb"], (r["unb"], se["unb"])
    assert r["bia"] < 0.75
    for bb in (1, 2):
        assert abs(r["mse%d" % bb] - (1 - oracle.lloyd_max(bb)[2])) < 0.02 + 5 * se["mse%d" % bb]
    assert r["mse1"] < r["res2"] < 1 - 5 * se["res2"]
    assert r["mse2"] < r["res3"] < 1 - 5 * se["res3"]


# ---------------------------------------------------------------- EDEN scale
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [16, 128])
def test_eden_scale_closed_form(bits, d):
    rng = np.random.default_rng(bits + d)
    x = rng.standard_normal((30, d)).astype(np.float32)
    x[0] = 0.0
    c, S = oracle.quantize_eden(x, bits, 61)
    c_mse, nr = oracle.quantize(x, bits, 61)
    np.testing.assert_array_equal(c, c_mse)                      # same codes as the MSE encoder
    assert S[0] == 0.0
    # <x^, x> = ||x||^2 for the decoded vector (decoder output rounded to fp32)
    xh = oracle.dequantize(c, S, d, bits, 61).astype(np.float64)
    x64 = x.astype(np.float64)
    np.testing.assert_allclose((xh * x64).sum(1)[1:], (x64 ** 2).sum(1)[1:], rtol=2e-6)
    # and S relates to the MSE scale through the per-vector shrink <x~, x> / ||x||^2
    xt = oracle.dequantize(c_mse, nr, d, bits, 61).astype(np.float64)
    shrink = (xt * x64).sum(1)[1:] / (x64 ** 2).sum(1)[1:]
    np.testing.assert_allclose(S[1:] * shrink, nr[1:], rtol=2e-6)


def test_eden_one_bit_is_drive_unbiased():
    rng = np.random.default_rng(77)
    d = 64
    x = rng.standard_normal((20, d)).astype(np.float32)
    c, S = oracle.quantize_eden(x, 1, 5)
    b, Sd = oracle.sign_quantize(x, True, 5)
    np.testing.assert_array_equal(c, b)
    np.testing.assert_allclose(oracle.dequantize(c, S, d, 1, 5), oracle.sign_dequantize(b, Sd, d, 5),
                               rtol=1e-5, atol=1e-6)


def test_eden_inner_products_unbiased_over_seeds():
    rng = np.random.default_rng(1)
    d, seeds = 64, range(1500)
    x = rng.standard_normal((1, d)).astype(np.float32)
    q = (x + 0.5 * rng.standard_normal((1, d))).astype(np.float32)
    true = float(x[0].astype(np.float64) @ q[0].astype(np.float64))
    for bits in (2, 3):
        v = []
        for s in seeds:
            c, S = oracle.quantize_eden(x, bits, s)
            v.append(oracle.score(q, c, S, d, bits, s)[0, 0])
        r, se = np.mean(v) / true, np.std(v) / np.sqrt(len(v)) / true
        assert abs(r - 1) < 5 * se + 2e-3, (bits, r, se)


# ------------------------------------------------- exact finite-d codebooks
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_beta_codebook_d3_is_the_uniform_quantizer(bits):
    # d = 3: a coordinate of a random unit vector is uniform on [-1, 1]
    K = 1 << bits
    lv, th, mse, _ = oracle.lloyd_max_beta(bits, 3)
    r3 = math.sqrt(3.0)
    np.testing.assert_allclose(lv, r3 * (-1 + (2 * np.arange(K) + 1) / K), atol=1e-10)
    np.testing.assert_allclose(th, r3 * (-1 + 2 * np.arange(1, K) / K), atol=1e-10)
    assert abs(mse - 1.0 / K ** 2) < 1e-10


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("d", [8, 64, 1024])
def test_beta_codebook_fixed_point_by_scipy(bits, d):
    # centroid and midpoint conditions under scipy's Beta law: (1 + y/sqrt d)/2 ~ Beta((d-1)/2, (d-1)/2);
    # the density is log-concave, so the Lloyd-Max fixed point is unique
    lv, th, mse, _ = oracle.lloyd_max_beta(bits, d)
    a, sd = (d - 1) / 2.0, math.sqrt(d)
    law = scipy.stats.beta(a, a)
    pdf = lambda y: law.pdf((1 + y / sd) / 2) / (2 * sd)
    edges = np.concatenate([[-sd], th, [sd]])
    np.testing.assert_allclose(th, (lv[1:] + lv[:-1]) / 2, atol=1e-12)
    err = 0.0
    for k in range(len(lv)):
        p = law.cdf((1 + edges[k + 1] / sd) / 2) - law.cdf((1 + edges[k] / sd) / 2)
        m1 = scipy.integrate.quad(lambda y: y * pdf(y), edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(m1 / p - lv[k]) < 1e-8, (k, m1 / p, lv[k])
        err += scipy.integrate.quad(lambda y: (y - lv[k]) ** 2 * pdf(y), edges[k], edges[k + 1],
                                    epsabs=1e-14, epsrel=1e-12)[0]
    assert abs(err - mse) < 1e-8


@pytest.mark.parametrize("d", [2, 5, 16, 128, 4096])
def test_beta_codebook_one_bit_closed_form(d):
    # 1 bit: the level is E|Y| = sqrt(d) E|t| = sqrt(d) Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    lv = oracle.lloyd_max_beta(1, d)[0]
    want = math.sqrt(d) * math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    np.testing.assert_allclose(lv, [-want, want], rtol=1e-11)


def test_beta_codebook_tends_to_the_normal_one():
    for bits in (1, 2, 3, 4):
        g = oracle.lloyd_max(bits)[0]
        b = oracle.lloyd_max_beta(bits, 1 << 16)[0]
        assert np.abs(b - g).max() < 2e-4
    # lighter tails at small d pull the outermost 3- and 4-bit levels in
    for bits in (3, 4):
        assert oracle.lloyd_max_beta(bits, 16)[0][-1] < oracle.lloyd_max(bits)[0][-1]


def test_given_codebook_codec_matches_the_normal_codec():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 64)).astype(np.float32)
    for bits in (1, 3, 4):
        lv, th, _, _ = oracle.lloyd_max(bits)
        c, n = oracle.quantize(x, bits, 9)
        cc, nn = oracle.quantize_cb(x, bits, 9, lv, th)
        np.testing.assert_array_equal(c, cc)
        np.testing.assert_array_equal(n, nn)
        np.testing.assert_array_equal(oracle.dequantize(c, n, 64, bits, 9), oracle.dequantize_cb(c, n, 64, bits, 9, lv))
