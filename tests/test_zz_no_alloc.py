"""rht_attention_noalloc (attention with the library's own device array in
place of a workspace) against rht_attention, both through the C ABI.

The two entry points run the same kernels with the same key chunking, so
their outputs must agree bit for bit; each is also held to the attention
error bound against the oracle's plain definition (tests/parity.py).  Two
calls in a row, the second smaller, check that what a call leaves in the
shared array does not leak into the next one.
"""
import sys

import numpy as np
import pytest
import scipy.linalg

import oracle
import rotation_vector_quantization_amd as rht
from parity import attention_bound, attention_terms

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

D = 128


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def coded(rng, heads, n, seed, bits):
    x = rng.standard_normal((heads * n, D)).astype(np.float32)
    x *= np.exp(0.5 * rng.standard_normal((heads * n, 1))).astype(np.float32)
    c, nr = oracle.quantize(x, bits, seed)
    return c.reshape(heads, n, -1), nr.reshape(heads, n)


def decoded(codes, norms, seed, bits):
    heads, n, _ = codes.shape
    out = oracle.dequantize(codes.reshape(heads * n, -1), norms.reshape(-1), D, bits, seed, np.float32)
    return out.reshape(heads, n, D).astype(np.float64)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def both(q, kc, kn, vc, vn, kb, vb, sk, sv, scale):
    """(noalloc output, workspace output) for one call each on the current stream."""
    heads, m, _ = q.shape
    n = kn.shape[1]
    qd, kcd, knd, vcd, vnd = dev(q), dev(kc), dev(kn), dev(vc), dev(vn)
    stream = torch.cuda.current_stream().cuda_stream
    out_na = torch.full((heads, m, D), float("nan"), dtype=torch.float32, device="cuda:0")
    rht.rht_attention_noalloc(qd.data_ptr(), m, kcd.data_ptr(), knd.data_ptr(), vcd.data_ptr(), vnd.data_ptr(),
                              heads, n, D, kb, vb, sk, sv, scale, out_na.data_ptr(), stream)
    need = rht.rht_attention_workspace_bytes(heads, m, n, D)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda:0")
    out_ws = torch.full((heads, m, D), float("nan"), dtype=torch.float32, device="cuda:0")
    rht.rht_attention(qd.data_ptr(), m, kcd.data_ptr(), knd.data_ptr(), vcd.data_ptr(), vnd.data_ptr(),
                      heads, n, D, kb, vb, sk, sv, scale, out_ws.data_ptr(), ws.data_ptr(), need, stream)
    torch.cuda.synchronize()
    return out_na.cpu().numpy(), out_ws.cpu().numpy()


def within_bound(got, q, kc, kn, vc, vn, kb, vb, sk, sv, scale):
    want = oracle.attention(q, kc, kn, vc, vn, D, kb, vb, sk, sv, scale)
    qt, kterm = attention_terms(q, kc, kn, D, kb, sk, oracle.lloyd_max(kb)[0],
                                oracle.signs(sk, D).astype(np.float64), scipy.linalg.hadamard(D))
    bound = attention_bound(q, qt, kterm, decoded(kc, kn, sk, kb), decoded(vc, vn, sv, vb), want, scale)
    err = np.linalg.norm(got.astype(np.float64) - want, axis=2)
    return float((err / bound).max())


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    rht.load()


def test_noalloc_matches_workspace_entry_two_calls():
    rng = np.random.default_rng(31)
    cases = [  # (heads, n, m, k_bits, v_bits): the second call is smaller than the first
        (40, 3000, 6, 4, 4),
        (3, 777, 3, 4, 3),
    ]
    for heads, n, m, kb, vb in cases:
        say("noalloc attention: heads=%d n=%d m=%d K%d/V%d" % (heads, n, m, kb, vb))
        kc, kn = coded(rng, heads, n, 5, kb)
        vc, vn = coded(rng, heads, n, 6, vb)
        q = rng.standard_normal((heads, m, D)).astype(np.float32)
        scale = 1.0 / np.sqrt(D)
        na, ws = both(q, kc, kn, vc, vn, kb, vb, 5, 6, scale)
        assert np.all(np.isfinite(na))
        np.testing.assert_array_equal(na.view(np.uint32), ws.view(np.uint32))
        worst = within_bound(na, q, kc, kn, vc, vn, kb, vb, 5, 6, scale)
        say("  bit-identical to rht_attention; worst error / bound %.3g" % worst)
        assert worst <= 1.0


def test_noalloc_rejects_sizes_beyond_its_array():
    heads, m, n = 4096, 16, 64
    assert rht.rht_attention_workspace_bytes(heads, m, n, D) > (32 << 20)
    t = torch.zeros(16, dtype=torch.uint8, device="cuda:0")
    p = t.data_ptr()
    with pytest.raises(rht.RhtError) as e:
        rht.rht_attention_noalloc(p, m, p, p, p, p, heads, n, D, 4, 4, 1, 2, 0.1, p,
                                  torch.cuda.current_stream().cuda_stream)
    assert e.value.status == 9  # RHT_E_WORKSPACE, before anything is queued
