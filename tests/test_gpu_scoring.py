"""GPU parity of scoring on sign-coded and residual-coded keys (rht_score_sign,
rht_residual_score, through the C ABI) against the CPU oracle on identical
code bytes produced by the oracle's encoders, at every d the encoders accept
(32 ... 4096; d >= 512 runs the query-group kernel), and at the sizes of the
scoring and the DRIVE workloads.  Rule: relative L2 <= SCORE_TOL
per query row and over all logits, as for MSE-coded keys; keys whose scale is
0 (zero vectors) must score exactly 0."""
import sys

import numpy as np
import pytest

import oracle
import rotation_vector_quantization_amd as rht
import testdata
from parity import SCORE_TOL, chunked, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def check(got, ref, what):
    nz = np.abs(ref).sum(0) > 0
    g = rel_l2(got[:, nz], ref[:, nz])
    per_row = rel_l2(got[:, nz], ref[:, nz], axis=1)
    say("%s: global rel L2 %.2e, worst query %.2e" % (what, g, per_row.max()))
    assert g <= SCORE_TOL and per_row.max() <= SCORE_TOL
    assert np.all(got[:, ~nz] == 0)


ALL_D = [16, 32, 64, 128, 256, 512, 1024, 2048, 4096]


@pytest.mark.parametrize("unbiased", [False, True])
@pytest.mark.parametrize("d", ALL_D)
@pytest.mark.parametrize("m,n", [(1, 1), (17, 100), (64, 1037), (33, 31), (40, 65), (32, 64)])
def test_sign_score_grid(unbiased, d, m, n):
    seed = 31 + d
    rng = np.random.default_rng(d * 7 + m + unbiased)
    keys = rng.standard_normal((n, d)).astype(np.float32)
    keys[0] = 0.0
    q = rng.standard_normal((m, d)).astype(np.float32)
    bits, S = oracle.sign_quantize(keys, unbiased, seed)
    say("sign score d=%d m=%d n=%d unbiased=%d" % (d, m, n, unbiased))
    got = host(rht.score_sign(dev(q), dev(bits), dev(S), d, seed))
    check(got, oracle.score_sign(q, bits, S, d, seed), "sign score")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", ALL_D)
@pytest.mark.parametrize("m,n", [(1, 1), (17, 100), (64, 1037), (33, 31), (40, 65), (32, 64)])
def test_residual_score_grid(bits, d, m, n):
    seed = 41 + d
    rng = np.random.default_rng(d * 11 + m + bits)
    keys = rng.standard_normal((n, d)).astype(np.float32)
    keys[0] = 0.0
    q = rng.standard_normal((m, d)).astype(np.float32)
    c, g, nr, rs = oracle.residual_quantize(keys, bits, seed)
    say("residual score d=%d bits=%d m=%d n=%d" % (d, bits, m, n))
    got = host(rht.residual_score(dev(q), dev(c), dev(g), dev(nr), dev(rs), d, bits, seed))
    check(got, oracle.score_residual(q, c, g, nr, rs, d, bits, seed), "residual score")


def test_sign_and_residual_scores_at_the_scoring_workload_size():
    # the scoring workload's shape: 131072 keys d=128, 64 queries
    wk, wq = testdata.WORKLOADS["c5k"], testdata.WORKLOADS["c5q"]
    keys = testdata.generate(wk)
    q = testdata.generate(wq)
    d, seed = wk.d, wk.rot_seed
    parts = chunked(lambda lo, hi: oracle.sign_quantize(keys[lo:hi], True, seed), wk.n)
    b = np.concatenate([p[0] for p in parts])
    S = np.concatenate([p[1] for p in parts])
    say("sign codes of the scoring keys from the oracle")
    got = host(rht.score_sign(dev(q), dev(b), dev(S), d, seed))
    ref = np.concatenate(chunked(lambda lo, hi: oracle.score_sign(q, b[lo:hi], S[lo:hi], d, seed), wk.n), axis=1)
    check(got, ref, "sign score, 131072 keys")
    parts = chunked(lambda lo, hi: oracle.residual_quantize(keys[lo:hi], 3, seed), wk.n)
    c, g, nr, rs = (np.concatenate([p[i] for p in parts]) for i in range(4))
    say("residual codes of the scoring keys from the oracle")
    got = host(rht.residual_score(dev(q), dev(c), dev(g), dev(nr), dev(rs), d, 3, seed))
    ref = np.concatenate(chunked(lambda lo, hi: oracle.score_residual(q, c[lo:hi], g[lo:hi], nr[lo:hi],
                                                                      rs[lo:hi], d, 3, seed), wk.n), axis=1)
    check(got, ref, "residual score, 131072 keys")


def test_sign_scores_of_the_drive_workload():
    """The DRIVE workload's own codes (65536 x 1024 Student-t rows, 1-bit signs
    with the unbiased scale) scored against 64 queries: d = 1024 runs the
    query-group kernel, 4 groups of 16 queries over every key."""
    w = testdata.WORKLOADS["c3"]
    x = testdata.generate(w)
    d, seed = w.d, w.rot_seed
    parts = chunked(lambda lo, hi: oracle.sign_quantize(x[lo:hi], True, seed), w.n)
    b = np.concatenate([p[0] for p in parts])
    S = np.concatenate([p[1] for p in parts])
    del x
    q = np.random.default_rng(1004).standard_normal((64, d)).astype(np.float32)
    say("sign codes of the DRIVE workload from the oracle")
    got = host(rht.score_sign(dev(q), dev(b), dev(S), d, seed))
    ref = np.concatenate(chunked(lambda lo, hi: oracle.score_sign(q, b[lo:hi], S[lo:hi], d, seed), w.n), axis=1)
    check(got, ref, "sign score, DRIVE workload (65536 keys d=1024)")
