"""The benchmark's streaming-ceiling kernels (rotation_vector_quantization_amd/
bench_kernels/stream_ceiling.hip): each writes exactly its outputs, with the
values its XOR fold defines, and nothing past them.  They carry no part of the
method; bench.py times them as the achievable ceiling of each traffic shape, so
this only checks that they touch the bytes they claim to.  Expected values are
the same folds computed with numpy on the seeded inputs."""
import ctypes
import os
import sys

import numpy as np
import pytest

import rotation_vector_quantization_amd.build as rb

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GUARD = 4096  # 32-bit words of sentinel past every output
SENTINEL = 0x7FC0BEEF


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    if not os.path.exists(rb.CEIL_LIB):
        pytest.fail("libstream_ceiling.so is not built (run rotation_vector_quantization_amd/build.py)")
    L = ctypes.CDLL(rb.CEIL_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.ceiling_encode_shape.argtypes = [vp, vp, vp, i64, i32, vp]
    L.ceiling_decode_shape.argtypes = [vp, vp, vp, i64, i32, vp]
    L.ceiling_score_shape.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    return L


def words(n, seed):
    return np.random.default_rng(seed).integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to("cuda:0")


def out_buffer(nwords):
    return torch.full((nwords + GUARD,), int(np.uint32(SENTINEL).view(np.int32)), dtype=torch.int32,
                      device="cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint32)


def check(got, want, what):
    n = want.size
    assert np.array_equal(got[:n], want), "%s: %d of %d words differ" % (what, int((got[:n] != want).sum()), n)
    assert np.all(got[n:] == SENTINEL), "%s: wrote past its output" % what


@pytest.mark.parametrize("n,bpc", [(16 * 700, 1), (16 * 700, 3), (16, 2)])
def test_encode_shape(lib, n, bpc):
    say("encode shape n=%d blocks/CU=%d" % (n, bpc))
    x = words(n * 64, 1 + n)                      # n fp16 rows of 256 B
    codes, scale = out_buffer(n * 16), out_buffer(n)
    xd = dev(x)
    assert lib.ceiling_encode_shape(xd.data_ptr(), codes.data_ptr(), scale.data_ptr(), n, bpc,
                                    torch.cuda.current_stream().cuda_stream) == 0
    # group g of 16 rows: lane l folds 16-byte chunks l, l + 64, l + 128, l + 192
    xc = x.reshape(n // 16, 4, 64, 4)
    o = xc[:, 0] ^ xc[:, 1] ^ xc[:, 2] ^ xc[:, 3]             # [g][lane][4]
    check(host(codes), o.reshape(-1), "codes")
    check(host(scale), (o[:, :16, 0] ^ o[:, :16, 3]).reshape(-1), "scales")


@pytest.mark.parametrize("n,bpc", [(16 * 700, 2), (16 * 700, 8), (16, 1)])
def test_decode_shape(lib, n, bpc):
    say("decode shape n=%d blocks/CU=%d" % (n, bpc))
    c, s = words(n * 16, 2 + n), words(n, 3 + n)
    y = out_buffer(n * 64)
    cd, sd = dev(c), dev(s)
    assert lib.ceiling_decode_shape(cd.data_ptr(), sd.data_ptr(), y.data_ptr(), n, bpc,
                                    torch.cuda.current_stream().cuda_stream) == 0
    cg = c.reshape(n // 16, 64, 4)                            # [g][lane][4]
    sv = s.reshape(n // 16, 16)[:, np.arange(64) // 4]       # lane l takes scale l / 4
    base = cg ^ sv[:, :, None]
    want = np.stack([base ^ np.uint32(k) for k in range(4)], axis=1)   # [g][k][lane][4]
    check(host(y), want.reshape(-1), "decoded rows")


@pytest.mark.parametrize("n,m,bpc", [(64 * 300, 64, 1), (64 * 300, 64, 3), (64 * 37, 40, 2), (64, 4, 1),
                                     (64 * 37, 1, 4)])
def test_score_shape(lib, n, m, bpc):
    say("score shape n=%d m=%d blocks/CU=%d" % (n, m, bpc))
    c, s = words(n * 16, 4 + n), words(n, 5 + n)
    logits = out_buffer(m * n)
    cd, sd = dev(c), dev(s)
    assert lib.ceiling_score_shape(cd.data_ptr(), sd.data_ptr(), logits.data_ptr(), n, m, bpc,
                                   torch.cuda.current_stream().cuda_stream) == 0
    g = n // 64
    cg = c.reshape(g, 4, 64, 4)
    o = cg[:, 0] ^ cg[:, 1] ^ cg[:, 2] ^ cg[:, 3]             # [g][lane][4]
    f = o[..., 0] ^ o[..., 1] ^ o[..., 2] ^ o[..., 3] ^ s.reshape(g, 64)   # [g][lane]
    want = np.empty((m, n), dtype=np.uint32)
    for half in range(2):
        for r in range(16):
            for h in range(2):
                q = 32 * half + 8 * (r // 4) + 4 * h + r % 4
                if q >= m:
                    continue
                fl = f[:, 32 * h:32 * h + 32]                # lanes i + 32 h, keys 64 g + i (+ 32)
                want[q].reshape(g, 64)[:, :32] = fl ^ np.uint32(r)
                want[q].reshape(g, 64)[:, 32:] = fl + np.uint32(r)
    check(host(logits), want.reshape(-1), "logits")


def test_rejects_bad_arguments(lib):
    buf = torch.empty(64 * 64, dtype=torch.int32, device="cuda:0")
    p, st = buf.data_ptr(), torch.cuda.current_stream().cuda_stream
    assert lib.ceiling_score_shape(p, p, p, 100, 64, 1, st) == -1       # n not a multiple of 64
    assert lib.ceiling_score_shape(p, p, p, 64, 65, 1, st) == -1        # m > 64
    assert lib.ceiling_score_shape(p, p, p, 64, 64, 0, st) == -1        # blocks per CU
    assert lib.ceiling_encode_shape(p, p, p, 24, 1, st) == -1           # n not a multiple of 16
    assert lib.ceiling_decode_shape(p, p, None, 16, 1, st) == -1        # null output
