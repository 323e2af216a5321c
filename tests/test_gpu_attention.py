"""GPU parity of attention over coded keys and values (rht_attention, through
the C ABI) against the CPU oracle's plain definition: decode K and V in fp64
(each with the codebook of its own width), softmax(scale q.k), weighted sum of
the decoded values.  Key and value widths run over 2, 3 and 4 bits, including
the KV-cache pairing of 4-bit keys with 3-bit values.

The coded inputs come from the oracle's encoder, or, at the full KV-block size,
from a seeded byte generator (any byte string is a valid 4-bit code row); no
input or expected value comes from the HIP path.  Tolerance: the error model
in tests/parity.py (attention_bound), per (head, query) output row; the kernel
splits every MFMA operand into fp16 hi + lo parts and accumulates in fp32, so
its error is fp32-level, scaled by how strongly the softmax depends on the
logits.  tests/test_attention_tolerance.py shows on the CPU that an emulation
of this arithmetic stays well inside the bound and that losing a lo part
leaves it.  Rows shaped like the benchmark's (m <= 4 queries, scale 1/sqrt(d))
are also held to relative L2 <= 1e-5, the tolerance for fp32 results; every
check prints the worst relative L2 it saw.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import rotation_vector_quantization_amd as rht
import scipy.linalg

from parity import attention_bound, attention_terms, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

D, BITS = 128, 4
WIDTHS = [(4, 4), (4, 3), (3, 3), (2, 2), (4, 2), (3, 4), (2, 4), (3, 2), (2, 3)]
BENCH_REL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    rht.load()
    return torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def coded(rng, heads, n, seed, row_scale=None, bits=BITS):
    x = rng.standard_normal((heads * n, D)).astype(np.float32)
    if row_scale is not None:
        x *= row_scale.reshape(-1, 1).astype(np.float32)
    c, nr = oracle.quantize(x, bits, seed)
    return c.reshape(heads, n, -1), nr.reshape(heads, n)


def widths(kc, vc):
    return kc.shape[-1] * 8 // D, vc.shape[-1] * 8 // D


def run(q, kc, kn, vc, vn, sk, sv, scale, workspace=None):
    kb, vb = widths(kc, vc)
    return host(rht.attention(dev(q), dev(kc), dev(kn), dev(vc), dev(vn), kb, vb, sk, sv, scale,
                              workspace=workspace))


def reference(q, kc, kn, vc, vn, sk, sv, scale):
    kb, vb = widths(kc, vc)
    return oracle.attention(q, kc, kn, vc, vn, D, kb, vb, sk, sv, scale)


def decoded(codes, norms, seed):
    heads, n, row = codes.shape
    out = oracle.dequantize(codes.reshape(heads * n, -1), norms.reshape(-1), D, row * 8 // D, seed, np.float32)
    return out.reshape(heads, n, D).astype(np.float64)


def check(got, want, what, q, kc, kn, vc, vn, sk, sv, scale, rel_max=None):
    heads, m, _ = want.shape
    kb, _ = widths(kc, vc)
    qt, kterm = attention_terms(q, kc, kn, D, kb, sk, oracle.lloyd_max(kb)[0],
                                oracle.signs(sk, D).astype(np.float64), scipy.linalg.hadamard(D))
    bound = attention_bound(q, qt, kterm, decoded(kc, kn, sk), decoded(vc, vn, sv), want, scale)
    err = np.linalg.norm(got.astype(np.float64) - want, axis=2)
    ref = np.linalg.norm(want, axis=2)
    rel = np.where(ref > 0, err / np.maximum(ref, 1e-300), 0.0)
    worst = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
    say("%s: worst row rel L2 %.3g; worst error / bound %.3g" % (
        what, rel.max(), (err / np.maximum(bound, 1e-300)).max()))
    assert np.all(err <= bound), "%s: row %s error %.3g > bound %.3g (rel L2 %.3g)" % (
        what, worst, err[worst], bound[worst], rel[worst])
    if rel_max is not None:
        assert rel.max() <= rel_max, "%s: worst row rel L2 %.3g > %.1g" % (what, rel.max(), rel_max)
    assert np.all(got[ref == 0] == 0), "%s: zero rows not exactly zero" % what
    assert np.all(np.isfinite(got))


# m <= 8 and m > 8 take different operand layouts: both sides of the switch are covered
@pytest.mark.parametrize("heads,m,n", [(1, 1, 1), (1, 4, 31), (3, 4, 32), (2, 16, 33), (3, 5, 100),
                                       (2, 8, 1000), (1, 4, 4099), (5, 3, 257), (1, 7, 40), (2, 9, 65)])
@pytest.mark.parametrize("scale", [1.0 / math.sqrt(D), 1.0])
@pytest.mark.parametrize("kb,vb", WIDTHS)
def test_attention_grid(heads, m, n, scale, kb, vb):
    rng = np.random.default_rng(heads * 1000 + m * 10 + n + 7 * kb + vb)
    kc, kn = coded(rng, heads, n, 51, bits=kb)
    vc, vn = coded(rng, heads, n, 52, bits=vb)
    q = (2 * rng.standard_normal((heads, m, D))).astype(np.float32)
    say("attention grid heads=%d m=%d n=%d scale=%g k_bits=%d v_bits=%d" % (heads, m, n, scale, kb, vb))
    want = reference(q, kc, kn, vc, vn, 51, 52, scale)
    bench_shaped = m <= 4 and scale < 1.0
    check(run(q, kc, kn, vc, vn, 51, 52, scale), want, "grid %d/%d/%d K%d/V%d" % (heads, m, n, kb, vb),
          q, kc, kn, vc, vn, 51, 52, scale, rel_max=BENCH_REL if bench_shaped else None)


@pytest.mark.parametrize("kb,vb", [(4, 4), (4, 3), (2, 2)])
@pytest.mark.parametrize("m", [4, 6, 12])   # one m per operand layout (<= 4, <= 8, <= 16)
def test_attention_degenerate_queries_and_values(m, kb, vb):
    rng = np.random.default_rng(3)
    heads, n = 4, 300
    kc, kn = coded(rng, heads, n, 61, bits=kb)
    vn_scale = np.ones(heads * n)
    vn_scale[:n] = 0.0                                           # head 0: every value is zero
    vn_scale[n:2 * n] = 10.0 ** rng.uniform(-20, 20, n)          # head 1: norms over 40 decades
    vn_scale[2 * n + 37] = 0.0                                   # head 2: one zero value
    vc, vn = coded(rng, heads, n, 62, vn_scale, bits=vb)
    q = rng.standard_normal((heads, m, D)).astype(np.float32)
    q[:, 0] = 0.0                                                # uniform weights
    q[:, 1] *= 1e4                                               # hard attention
    q[:, 2] *= 1e-30                                             # tiny query
    say("attention degenerate cases m=%d k_bits=%d v_bits=%d" % (m, kb, vb))
    want = reference(q, kc, kn, vc, vn, 61, 62, 1.0 / math.sqrt(D))
    got = run(q, kc, kn, vc, vn, 61, 62, 1.0 / math.sqrt(D))
    assert np.all(got[0] == 0.0)
    check(got, want, "degenerate", q, kc, kn, vc, vn, 61, 62, 1.0 / math.sqrt(D))


def test_attention_workspace_reused_by_a_smaller_call():
    rng = np.random.default_rng(4)
    big = (6, 8, 2000)
    need = rht.rht_attention_workspace_bytes(*big, D)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda:0")
    for heads, m, n in (big, (2, 3, 77)):
        kc, kn = coded(rng, heads, n, 71)
        vc, vn = coded(rng, heads, n, 72)
        q = rng.standard_normal((heads, m, D)).astype(np.float32)
        say("attention with a shared workspace heads=%d m=%d n=%d" % (heads, m, n))
        want = reference(q, kc, kn, vc, vn, 71, 72, 0.1)
        check(run(q, kc, kn, vc, vn, 71, 72, 0.1, workspace=ws), want, "shared workspace",
              q, kc, kn, vc, vn, 71, 72, 0.1)


@pytest.mark.parametrize("m,kb,vb", [(4, 4, 4), (8, 4, 4), (16, 4, 4), (4, 4, 3)])
def test_attention_kv_block_full_size_sampled_heads(m, kb, vb):
    # the benchmark's shape: 32 layers x 8 KV heads = 256 heads, 32768 tokens;
    # the benchmark's m = 4 with the other two operand layouts, and 4-bit keys
    # with 3-bit values (any byte string is a valid row of b-bit codes)
    heads, n = 256, 32768
    rng = np.random.default_rng(20250)
    kc = rng.integers(0, 256, (heads, n, kb * D // 8), dtype=np.uint8)
    vc = rng.integers(0, 256, (heads, n, vb * D // 8), dtype=np.uint8)
    kn = np.exp(0.5 * rng.standard_normal((heads, n))).astype(np.float32) * math.sqrt(D)
    vn = np.exp(0.5 * rng.standard_normal((heads, n))).astype(np.float32) * math.sqrt(D)
    q = rng.standard_normal((heads, m, D)).astype(np.float32)
    say("attention full size: %d heads x %d keys x %d queries, K%d/V%d" % (heads, n, m, kb, vb))
    got = run(q, kc, kn, vc, vn, 42, 43, 1.0 / math.sqrt(D))
    assert np.all(np.isfinite(got))
    for h in (0, 77, 255):
        want = reference(q[h:h + 1], kc[h:h + 1], kn[h:h + 1], vc[h:h + 1], vn[h:h + 1], 42, 43, 1.0 / math.sqrt(D))
        check(got[h:h + 1], want, "full size head %d" % h, q[h:h + 1], kc[h:h + 1], kn[h:h + 1],
              vc[h:h + 1], vn[h:h + 1], 42, 43, 1.0 / math.sqrt(D), rel_max=BENCH_REL if m <= 4 else None)


@pytest.mark.parametrize("kb,vb", [(4, 4), (4, 3), (3, 2)])
@pytest.mark.parametrize("m", [1, 4, 5, 8, 9, 16])   # both sides of every operand-layout switch
def test_attention_key_counts_and_buffer_bounds(m, kb, vb):
    """Key counts on and around the 32-key tiles and the per-head chunking, through
    the raw C ABI: the output [heads][m][d] and the workspace carry sentinel bytes
    past their ends (the workspace past rht_attention_workspace_bytes), which must
    survive; the output must meet the error bound."""
    heads, sk, sv, scale = 2, 81, 82, 1.0 / math.sqrt(D)
    rng = np.random.default_rng(300 + m + 10 * kb + vb)
    for n in (1, 2, 31, 32, 33, 63, 64, 65, 1023, 1025, 3073):
        say("attention key counts heads=%d m=%d n=%d K%d/V%d" % (heads, m, n, kb, vb))
        kc, kn = coded(rng, heads, n, sk, bits=kb)
        vc, vn = coded(rng, heads, n, sv, bits=vb)
        q = (2 * rng.standard_normal((heads, m, D))).astype(np.float32)
        ob = heads * m * D * 4
        need = rht.rht_attention_workspace_bytes(heads, m, n, D)
        out = torch.full((ob + 4096,), 0xA5, dtype=torch.uint8, device="cuda:0")
        ws = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device="cuda:0")
        qd, kcd, knd, vcd, vnd = dev(q), dev(kc), dev(kn), dev(vc), dev(vn)
        rht.rht_attention(qd.data_ptr(), m, kcd.data_ptr(), knd.data_ptr(), vcd.data_ptr(), vnd.data_ptr(),
                          heads, n, D, kb, vb, sk, sv, scale, out.data_ptr(), ws.data_ptr(), need,
                          torch.cuda.current_stream().cuda_stream)
        o, w = host(out), host(ws)
        assert np.all(o[ob:] == 0xA5), "attention wrote past its output"
        assert np.all(w[need:] == 0xA5), "attention wrote past its workspace"
        want = reference(q, kc, kn, vc, vn, sk, sv, scale)
        check(o[:ob].view(np.float32).reshape(heads, m, D), want, "key counts m=%d n=%d" % (m, n),
              q, kc, kn, vc, vn, sk, sv, scale)
