"""GPU parity at row counts on and around the kernels' tile edges (wave tiles of
16 rows, blocks of 64 rows, and their multiples), through the raw C ABI with
output buffers longer than n: every row past n must keep its sentinel bytes,
and the first n rows must match the oracle under the rules of tests/parity.py.
"""
import numpy as np
import pytest

import oracle
import rotation_vector_quantization_amd as rht
from parity import (RECON_F16, RECON_F32, NORM_RTOL, SCALE_RTOL, check_codes, check_recon, check_rel,
                    unpack)
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
@pytest.mark.parametrize("d,dt", [(128, np.float16), (128, np.float32), (256, np.float16), (1024, np.float32)])
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


@pytest.mark.parametrize("mode", [rht.SCALE_SIGN_BIASED, rht.SCALE_SIGN_UNBIASED])
def test_drive_row_counts(mode):
    d, dt, seed = 1024, np.float32, 77
    X = small_input(max(EDGES), d, dt, seed)
    for n in EDGES:
        say("drive row counts mode=%d n=%d" % (mode, n))
        x = X[:n]
        xd = to_dev(x)
        bits, S = padded(n, d // 8), padded(n, 4)
        rht.rht_quantize(xd.data_ptr(), rht.F32, n, d, 1, mode, seed, bits.data_ptr(), S.data_ptr(), stream())
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
@pytest.mark.parametrize("d,dt", [(256, np.float16), (128, np.float32)])
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
