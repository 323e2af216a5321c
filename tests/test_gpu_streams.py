"""The stream argument of every entry point: work queued on two side streams at
once, and the same calls captured in a HIP graph and replayed, must give the
bytes that the default stream gives.  The library's entry points only launch
kernels (no allocation, copy, memset or synchronisation), so both must hold
exactly; the kernels are deterministic (no atomics, fixed reduction order).
Inputs are seeded; the default-stream results are themselves checked against
the oracle by the parity tests.
"""
import sys

import numpy as np
import pytest

import oracle
import rotation_vector_quantization_amd as rht

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

D, BITS = 128, 4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    rht.load()


def kv_input(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)) * np.exp(0.5 * rng.standard_normal((n, 1)))
    return torch.from_numpy(x.astype(np.float16)).to("cuda:0")


def pipeline(x, q, seed):
    """Encode, decode, score and attend (keys = values = the coded rows, one head)."""
    codes, norms = rht.quantize(x, BITS, seed)
    y = rht.dequantize(codes, norms, D, BITS, seed, dtype=torch.float16)
    logits = rht.score(q, codes, norms, D, BITS, seed)
    n = x.shape[0]
    att = rht.attention(q[None], codes.view(1, n, -1), norms.view(1, n), codes.view(1, n, -1),
                        norms.view(1, n), BITS, BITS, seed, seed, 0.1)
    return [codes, norms, y, logits, att]


def same(a, b, what):
    for i, (u, v) in enumerate(zip(a, b)):
        assert torch.equal(u, v), "%s: output %d differs" % (what, i)


def test_two_side_streams_match_the_default_stream():
    xa, xb = kv_input(20000, 1), kv_input(30001, 2)
    q = torch.randn((8, D), generator=torch.Generator().manual_seed(3)).to("cuda:0")
    ref_a, ref_b = pipeline(xa, q, 11), pipeline(xb, q, 12)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        say("side streams, repetition %d" % rep)
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            got_a = pipeline(xa, q, 11)
        with torch.cuda.stream(s2):
            got_b = pipeline(xb, q, 12)
        torch.cuda.synchronize()
        same(got_a, ref_a, "stream 1")
        same(got_b, ref_b, "stream 2")


def test_graph_replays_match_eager_calls():
    n, seed = 12345, 21
    x = kv_input(n, 5)
    q = torch.randn((4, D), generator=torch.Generator().manual_seed(6)).to("cuda:0")
    codes = torch.empty((n, D * BITS // 8), dtype=torch.uint8, device="cuda:0")
    norms = torch.empty((n,), dtype=torch.float32, device="cuda:0")
    y = torch.empty((n, D), dtype=torch.float16, device="cuda:0")
    logits = torch.empty((4, n), dtype=torch.float32, device="cuda:0")
    att = torch.empty((1, 4, D), dtype=torch.float32, device="cuda:0")
    need = rht.rht_attention_workspace_bytes(1, 4, n, D)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda:0")

    def calls():
        st = torch.cuda.current_stream().cuda_stream
        rht.rht_quantize(x.data_ptr(), rht.F16, n, D, BITS, rht.SCALE_NORM, seed, codes.data_ptr(),
                         norms.data_ptr(), st)
        rht.rht_dequantize(codes.data_ptr(), norms.data_ptr(), n, D, BITS, rht.SCALE_NORM, seed, y.data_ptr(),
                           rht.F16, st)
        rht.rht_score(q.data_ptr(), 4, codes.data_ptr(), norms.data_ptr(), n, D, BITS, seed, logits.data_ptr(), st)
        rht.rht_attention(q.data_ptr(), 4, codes.data_ptr(), norms.data_ptr(), codes.data_ptr(), norms.data_ptr(),
                          1, n, D, BITS, BITS, seed, seed, 0.1, att.data_ptr(), ws.data_ptr(), need, st)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # first calls outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        say("graph replay %d" % rep)
        x.copy_(kv_input(n, 100 + rep))  # new input, eager, between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (codes, norms, y, logits, att)]
        calls()  # the same calls, eager
        torch.cuda.synchronize()
        same(got, [codes, norms, y, logits, att], "replay %d" % rep)
        # and the replay computed this input, not a stale one
        c0 = oracle.quantize(x[:64].cpu().numpy(), BITS, seed)[0]
        assert (got[0][:64].cpu().numpy() != c0).mean() < 1e-3
