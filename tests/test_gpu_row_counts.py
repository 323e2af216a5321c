"""GPU parity at row counts on and around the kernels' tile edges (wave tiles of
16 rows, blocks of 64 rows, 32-key scoring tiles, and their multiples), through
the raw C ABI with output buffers longer than needed: every byte past the
output must keep its sentinel value, and the output must match the oracle
under the rules of tests/parity.py.
"""
import numpy as np
import pytest

import oracle
import rotation_vector_quantization_amd as rht
from parity import (RECON_F16, RECON_F32, NORM_RTOL, SCALE_RTOL, SCORE_TOL, check_codes, check_recon,
                    check_rel, rel_l2, unpack)
from test_gpu_parity import check_residual, small_input, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EDGES = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1023, 1024, 1025]
PAD = 67        # sentinel rows past n in every output buffer
SENT = 0xA5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    rht.load()


def stream():
    return torch.cuda.current_stream().cuda_stream


def padded(n, row_bytes):
    """A device byte buffer of n + PAD rows, filled with the sentinel."""
    return torch.full(((n + PAD) * row_bytes,), SENT, dtype=torch.uint8, device="cuda:0")


def split(buf, n, row_bytes, dtype=np.uint8):
    """Host copy of the first n rows (as `dtype`), after checking the rows past n."""
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[n * row_bytes:] == SENT), "a kernel wrote past row n = %d" % n
    return b[:n * row_bytes].view(dtype).reshape(n, -1)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def xcode(dt):
    return rht.F16 if dt == np.float16 else rht.F32


@pytest.mark.parametrize("bits", [1, 3, 4])
@pytest.mark.parametrize("d,dt", [(16, np.float16), (16, np.float32), (128, np.float16), (128, np.float32),
                                  (256, np.float16), (1024, np.float32)])
def test_mse_row_counts(d, dt, bits):
    seed = 500 + d + bits
    X = small_input(max(EDGES), d, dt, seed)
    _, th, _, _ = oracle.lloyd_max(bits)
    cb = d * bits // 8
    for n in EDGES:
        say("mse row counts d=%d bits=%d x=%s n=%d" % (d, bits, np.dtype(dt).name, n))
        x = X[:n]
        xd = to_dev(x)
        codes, scale = padded(n, cb), padded(n, 4)
        rht.rht_quantize(xd.data_ptr(), xcode(dt), n, d, bits, rht.SCALE_NORM, seed, codes.data_ptr(),
                         scale.data_ptr(), stream())
        gc, gs = split(codes, n, cb), split(scale, n, 4, np.float32)[:, 0]
        oc, os_ = oracle.quantize(x, bits, seed)
        check_codes(unpack(gc, bits, d), unpack(oc, bits, d),
                    lambda rows: oracle.quantize(x[rows], bits, seed, want_y=True)[2], th, "codes")
        check_rel(gs, os_, NORM_RTOL, "norms")
        for yt, ydt, tol in ((rht.F16, np.float16, RECON_F16), (rht.F32, np.float32, RECON_F32)):
            yb = np.dtype(ydt).itemsize * d
            y = padded(n, yb)
            rht.rht_dequantize(codes.data_ptr(), scale.data_ptr(), n, d, bits, rht.SCALE_NORM, seed,
                               y.data_ptr(), yt, stream())
            check_recon(split(y, n, yb, ydt), oracle.dequantize(gc, gs, d, bits, seed, ydt), tol,
                        "dequant %s" % np.dtype(ydt).name)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("mode", [rht.SCALE_EDEN, rht.SCALE_NORM_BETA])
@pytest.mark.parametrize("d,dt", [(16, np.float16), (128, np.float16), (1024, np.float32)])
def test_eden_and_finite_d_row_counts(d, dt, mode, bits):
    seed = 700 + d + bits + mode
    X = small_input(max(EDGES), d, dt, seed)
    if mode == rht.SCALE_EDEN:
        lv, th, _, _ = oracle.lloyd_max(bits)
    else:
        lv, th, _, _ = oracle.lloyd_max_beta(bits, d)
    cb = d * bits // 8
    for n in EDGES:
        say("%s row counts d=%d bits=%d n=%d" % ("eden" if mode == rht.SCALE_EDEN else "beta", d, bits, n))
        x = X[:n]
        xd = to_dev(x)
        codes, scale = padded(n, cb), padded(n, 4)
        rht.rht_quantize(xd.data_ptr(), xcode(dt), n, d, bits, mode, seed, codes.data_ptr(), scale.data_ptr(),
                         stream())
        gc, gs = split(codes, n, cb), split(scale, n, 4, np.float32)[:, 0]
        if mode == rht.SCALE_EDEN:
            oc, os_ = oracle.quantize_eden(x, bits, seed)
            ys = lambda rows: oracle.quantize(x[rows], bits, seed, want_y=True)[2]
        else:
            oc, os_ = oracle.quantize_cb(x, bits, seed, lv, th)
            ys = lambda rows: oracle.quantize_cb(x[rows], bits, seed, lv, th, want_y=True)[2]
        gu, ou = unpack(gc, bits, d), unpack(oc, bits, d)
        check_codes(gu, ou, ys, th, "codes")
        same = (gu == ou).all(1)  # EDEN's S sums over every code of its row
        check_rel(gs[same], os_[same], SCALE_RTOL if mode == rht.SCALE_EDEN else NORM_RTOL, "scale")
        y = padded(n, 4 * d)
        rht.rht_dequantize(codes.data_ptr(), scale.data_ptr(), n, d, bits, mode, seed, y.data_ptr(), rht.F32,
                           stream())
        ref = oracle.dequantize_cb(gc, gs, d, bits, seed, lv, np.float32)
        check_recon(split(y, n, 4 * d, np.float32), ref, RECON_F32, "decode")


@pytest.mark.parametrize("mode", [rht.SCALE_SIGN_BIASED, rht.SCALE_SIGN_UNBIASED])
@pytest.mark.parametrize("d,dt", [(16, np.float16), (1024, np.float32)])
def test_drive_row_counts(d, dt, mode):
    seed = 77
    X = small_input(max(EDGES), d, dt, seed)
    for n in EDGES:
        say("drive row counts d=%d mode=%d n=%d" % (d, mode, n))
        x = X[:n]
        xd = to_dev(x)
        bits, S = padded(n, d // 8), padded(n, 4)
        rht.rht_quantize(xd.data_ptr(), xcode(dt), n, d, 1, mode, seed, bits.data_ptr(), S.data_ptr(), stream())
        gb, gS = split(bits, n, d // 8), split(S, n, 4, np.float32)[:, 0]
        ob, oS = oracle.sign_quantize(x, mode == rht.SCALE_SIGN_UNBIASED, seed)
        check_codes(unpack(gb, 1, d), unpack(ob, 1, d),
                    lambda rows: oracle.sign_quantize(x[rows], False, seed, want_y=True)[2],
                    np.array([0.0]), "drive bits")
        check_rel(gS, oS, SCALE_RTOL, "S")
        y = padded(n, 4 * d)
        rht.rht_dequantize(bits.data_ptr(), S.data_ptr(), n, d, 1, mode, seed, y.data_ptr(), rht.F32, stream())
        check_recon(split(y, n, 4 * d, np.float32), oracle.sign_dequantize(gb, gS, d, seed, np.float32),
                    RECON_F32, "drive decode")


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("d,dt", [(16, np.float16), (16, np.float32), (256, np.float16), (128, np.float32)])
def test_residual_row_counts(d, dt, bits):
    seed = 900 + d + bits
    X = small_input(max(EDGES), d, dt, seed)
    cb, sb = d * (bits - 1) // 8, d // 8
    for n in EDGES:
        say("residual row counts d=%d bits=%d x=%s n=%d" % (d, bits, np.dtype(dt).name, n))
        x = X[:n]
        xd = to_dev(x)
        codes, sg, norms, rs = padded(n, cb), padded(n, sb), padded(n, 4), padded(n, 4)
        rht.rht_residual_quantize(xd.data_ptr(), xcode(dt), n, d, bits, seed, codes.data_ptr(), sg.data_ptr(),
                                  norms.data_ptr(), rs.data_ptr(), stream())
        gc, gsg = split(codes, n, cb), split(sg, n, sb)
        gn, grs = split(norms, n, 4, np.float32)[:, 0], split(rs, n, 4, np.float32)[:, 0]
        check_residual(x, bits, seed, gc, gsg, gn, grs)
        for yt, ydt, tol in ((rht.F16, np.float16, RECON_F16), (rht.F32, np.float32, RECON_F32)):
            yb = np.dtype(ydt).itemsize * d
            y = padded(n, yb)
            rht.rht_residual_dequantize(codes.data_ptr(), sg.data_ptr(), norms.data_ptr(), rs.data_ptr(), n, d,
                                        bits, seed, y.data_ptr(), yt, stream())
            ref = oracle.residual_dequantize(gc, gsg, gn, grs, d, bits, seed, ydt)
            check_recon(split(y, n, yb, ydt), ref, tol, "residual decode %s" % np.dtype(ydt).name)


SCORE_N = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1025]


@pytest.mark.parametrize("kind", ["mse4", "mse2", "sign", "res3"])
@pytest.mark.parametrize("m", [1, 32, 33, 64])
@pytest.mark.parametrize("d", [16, 32, 64, 128, 1024])
def test_score_key_counts(d, m, kind):
    """Logits [m][n] for key counts around the 32-key tiles and 64-key items; the
    buffer carries sentinel bytes past m * n.  Every logit <q, k^> must be within
    SCORE_TOL * ||q|| * ||k^|| of the oracle's (the Cauchy-Schwarz scale of the
    dot product; k^ is the decoded key); the relative-L2 rules, overall and per
    query row, apply once a row holds a whole 32-key tile, since over one or two
    logits a relative error measures only the cancellation inside a dot product."""
    seed = 60 + d + m
    rng = np.random.default_rng(d + 3 * m + len(kind))
    K = rng.standard_normal((max(SCORE_N), d)).astype(np.float32)
    K[0] = 0.0
    q = rng.standard_normal((m, d)).astype(np.float32)
    qd = to_dev(q)
    for n in SCORE_N:
        say("score key counts d=%d m=%d kind=%s n=%d" % (d, m, kind, n))
        keys = K[:n]
        out = torch.full((m * n * 4 + PAD * 256,), SENT, dtype=torch.uint8, device="cuda:0")
        if kind.startswith("mse"):
            bits = int(kind[3:])
            c, nr = oracle.quantize(keys, bits, seed)
            cd, nd = to_dev(c), to_dev(nr)
            rht.rht_score(qd.data_ptr(), m, cd.data_ptr(), nd.data_ptr(), n, d, bits, seed, out.data_ptr(), stream())
            ref = oracle.score(q, c, nr, d, bits, seed)
            khat = oracle.dequantize(c, nr, d, bits, seed, np.float32)
        elif kind == "sign":
            b, S = oracle.sign_quantize(keys, True, seed)
            bd, Sd = to_dev(b), to_dev(S)
            rht.rht_score_sign(qd.data_ptr(), m, bd.data_ptr(), Sd.data_ptr(), n, d, seed, out.data_ptr(), stream())
            ref = oracle.score_sign(q, b, S, d, seed)
            khat = oracle.sign_dequantize(b, S, d, seed, np.float32)
        else:
            bits = int(kind[3:])
            c, g, nr, rs = oracle.residual_quantize(keys, bits, seed)
            cd, gd, nd, rd = to_dev(c), to_dev(g), to_dev(nr), to_dev(rs)
            rht.rht_residual_score(qd.data_ptr(), m, cd.data_ptr(), gd.data_ptr(), nd.data_ptr(), rd.data_ptr(), n,
                                   d, bits, seed, out.data_ptr(), stream())
            ref = oracle.score_residual(q, c, g, nr, rs, d, bits, seed)
            khat = oracle.residual_dequantize(c, g, nr, rs, d, bits, seed, np.float32)
        torch.cuda.synchronize()
        b = out.cpu().numpy()
        assert np.all(b[m * n * 4:] == SENT), "scoring wrote past m * n logits"
        got = b[:m * n * 4].view(np.float32).reshape(m, n)
        nz = np.abs(ref).sum(0) > 0
        assert np.all(got[:, ~nz] == 0)
        scale = np.linalg.norm(q.astype(np.float64), axis=1)[:, None] * \
            np.linalg.norm(khat.astype(np.float64), axis=1)[None, :]
        assert np.all(np.abs(got.astype(np.float64) - ref) <= SCORE_TOL * scale)
        if n >= 32:
            assert rel_l2(got[:, nz], ref[:, nz]) <= SCORE_TOL
            assert rel_l2(got[:, nz], ref[:, nz], axis=1).max() <= SCORE_TOL
