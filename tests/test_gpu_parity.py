"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on the
same seeded inputs.  Comparison rules are in tests/parity.py.

Small grids cover every kernel instantiation family with ragged row counts
(several blocks plus a partial tail) and the degenerate rows (zero vector,
exact zeros after rotation, one-hot rows); the workload tests run the full
sizes of the five workloads with the launch configuration the benchmark
times, checking every row where the oracle can afford it and a seeded sample
of rows elsewhere.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import rotation_vector_quantization_amd as rht
import testdata
from parity import (RECON_F16, RECON_F32, NORM_RTOL, SCALE_RTOL, SCORE_TOL, NEAR_REL,
                    MAX_NEAR_FRAC, check_codes, check_recon, check_recon_all, check_rel, chunked, rel_l2,
                    unpack)

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


def np_dtype(name):
    return np.float16 if name == "f16" else np.float32


def tdtype(name):
    return torch.float16 if name == "f16" else torch.float32


def special_rows(d, seed, dt):
    """Zero row, a row whose rotation has exact zeros, a one-hot row."""
    s = oracle.signs(seed, d)
    z = np.zeros((3, d), np.float64)
    z[1, 0], z[1, 1] = s[0] * 0.5, s[1] * 0.5  # H D x = H (e0 + e1)/2: half the coords are 0
    z[2, d // 3] = -3.0
    return z.astype(dt)


def small_input(n, d, dt, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    x[:, rng.choice(d, size=max(1, d // 64), replace=False)] *= 20.0
    x *= np.exp(0.5 * rng.standard_normal((n, 1)))
    x = x.astype(dt)
    x[:3] = special_rows(d, seed, dt)
    return x


def gpu_quantize(x, bits, seed, mode=0):
    codes, scale = rht.quantize(dev(x), bits, seed, mode)
    return host(codes), host(scale)


# ------------------------------------------------------------------ MSE code
@pytest.mark.parametrize("xdt", ["f32", "f16"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_mse_roundtrip_grid(d, bits, xdt):
    n = 777 if d <= 512 else 203
    seed = 1000 + d + bits
    say("mse grid d=%d bits=%d x=%s n=%d" % (d, bits, xdt, n))
    x = small_input(n, d, np_dtype(xdt), seed)
    codes, norms = gpu_quantize(x, bits, seed)
    ocodes, onorms = oracle.quantize(x, bits, seed)
    _, th, _, _ = oracle.lloyd_max(bits)
    check_codes(unpack(codes, bits, d), unpack(ocodes, bits, d),
                lambda rows: oracle.quantize(x[rows], bits, seed, want_y=True)[2], th, "codes")
    check_rel(norms, onorms, NORM_RTOL, "norms")
    assert np.all(unpack(codes[:1], bits, d) == (1 << bits) // 2) and norms[0] == 0
    for odt, tol in (("f32", RECON_F32), ("f16", RECON_F16)):
        y = host(rht.dequantize(dev(codes), dev(norms), d, bits, seed, dtype=tdtype(odt)))
        ref = oracle.dequantize(codes, norms, d, bits, seed, np_dtype(odt))
        check_recon(y, ref, tol, "dequant %s" % odt)


# ------------------------------------------------------------------ EDEN scale
@pytest.mark.parametrize("xdt", ["f32", "f16"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [16, 32, 128, 256, 1024, 4096])
def test_eden_grid(d, bits, xdt):
    n = 555 if d <= 1024 else 131
    seed = 3000 + d + bits
    say("eden grid d=%d bits=%d x=%s n=%d" % (d, bits, xdt, n))
    x = small_input(n, d, np_dtype(xdt), seed)
    codes, S = gpu_quantize(x, bits, seed, rht.SCALE_EDEN)
    ocodes, oS = oracle.quantize_eden(x, bits, seed)
    _, th, _, _ = oracle.lloyd_max(bits)
    gc, oc = unpack(codes, bits, d), unpack(ocodes, bits, d)
    check_codes(gc, oc, lambda rows: oracle.quantize(x[rows], bits, seed, want_y=True)[2], th, "eden codes")
    # S sums over every code of its row: compare it on rows whose codes all agree
    same = (gc == oc).all(1)
    check_rel(S[same], oS[same], SCALE_RTOL, "eden S")
    assert S[0] == 0
    for odt, tol in (("f32", RECON_F32), ("f16", RECON_F16)):
        y = host(rht.dequantize(dev(codes), dev(S), d, bits, seed, rht.SCALE_EDEN, dtype=tdtype(odt)))
        ref = oracle.dequantize(codes, S, d, bits, seed, np_dtype(odt))
        check_recon(y, ref, tol, "eden decode %s" % odt)


# ------------------------------------------------------------------ finite-d codebook
@pytest.mark.parametrize("xdt", ["f32", "f16"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [16, 32, 128, 1024])
def test_beta_codebook_grid(d, bits, xdt):
    # d = 128, fp16, 4 bits runs the MFMA KV-block kernels with this codebook
    n = 555
    seed = 4000 + d + bits
    say("finite-d codebook grid d=%d bits=%d x=%s" % (d, bits, xdt))
    x = small_input(n, d, np_dtype(xdt), seed)
    lv, th, _, _ = oracle.lloyd_max_beta(bits, d)
    codes, norms = gpu_quantize(x, bits, seed, rht.SCALE_NORM_BETA)
    ocodes, onorms = oracle.quantize_cb(x, bits, seed, lv, th)
    check_codes(unpack(codes, bits, d), unpack(ocodes, bits, d),
                lambda rows: oracle.quantize_cb(x[rows], bits, seed, lv, th, want_y=True)[2], th, "beta codes")
    check_rel(norms, onorms, NORM_RTOL, "norms")
    for odt, tol in (("f32", RECON_F32), ("f16", RECON_F16)):
        y = host(rht.dequantize(dev(codes), dev(norms), d, bits, seed, rht.SCALE_NORM_BETA, dtype=tdtype(odt)))
        ref = oracle.dequantize_cb(codes, norms, d, bits, seed, lv, np_dtype(odt))
        check_recon(y, ref, tol, "beta decode %s" % odt)


# ------------------------------------------------------------------ DRIVE
@pytest.mark.parametrize("mode", [rht.SCALE_SIGN_BIASED, rht.SCALE_SIGN_UNBIASED])
@pytest.mark.parametrize("xdt", ["f32", "f16"])
@pytest.mark.parametrize("d", [16, 32, 128, 1024, 4096])
def test_drive_grid(d, xdt, mode):
    n = 555 if d <= 1024 else 131
    seed = 77 + d
    say("drive grid d=%d x=%s mode=%d" % (d, xdt, mode))
    rng = np.random.default_rng(d)
    x = rng.standard_t(3, size=(n, d)).astype(np_dtype(xdt))
    x[:3] = special_rows(d, seed, np_dtype(xdt))
    b, S = gpu_quantize(x, 1, seed, mode)
    ob, oS = oracle.sign_quantize(x, mode == rht.SCALE_SIGN_UNBIASED, seed)
    check_codes(unpack(b, 1, d), unpack(ob, 1, d),
                lambda rows: oracle.sign_quantize(x[rows], False, seed, want_y=True)[2],
                np.array([0.0]), "drive bits")
    check_rel(S, oS, SCALE_RTOL, "S")
    assert S[0] == 0
    for odt, tol in (("f32", RECON_F32), ("f16", RECON_F16)):
        y = host(rht.dequantize(dev(b), dev(S), d, 1, seed, mode, dtype=tdtype(odt)))
        ref = oracle.sign_dequantize(b, S, d, seed, np_dtype(odt))
        check_recon(y, ref, tol, "drive decode %s" % odt)


# ------------------------------------------------------------------ residual chain
def check_residual(x, bits, seed, codes, sg, norms, rs, rows=None, what="residual"):
    """Compare GPU residual outputs (for `rows`, default all) with the oracle.
    Stage-1 codes against the oracle's own; sign bits and S_r against the
    oracle run on the GPU's stage-1 codes."""
    d = x.shape[1]
    if rows is None:
        rows = np.arange(x.shape[0])
    xs = x if len(rows) == x.shape[0] else x[rows]
    ocodes, _, onorms, _ = oracle.residual_quantize(xs, bits, seed)
    _, th1, _, _ = oracle.lloyd_max(bits - 1)
    lv1, _, _, _ = oracle.lloyd_max(bits - 1)
    gcodes = unpack(codes[rows], bits - 1, d)
    check_codes(gcodes, unpack(ocodes, bits - 1, d),
                lambda r: oracle.quantize(xs[r], bits - 1, seed, want_y=True)[2], th1, what + " stage 1")
    check_rel(norms[rows], onorms, NORM_RTOL, what + " norms")
    _, fsg, _, frs, fy = oracle.residual_quantize(xs, bits, seed, forced_codes=codes[rows], want_y=True)
    gs, os_ = unpack(sg[rows], 1, d), unpack(fsg, 1, d)
    mism = np.nonzero(gs != os_)
    if mism[0].size:
        c = lv1[gcodes[mism]]
        near = np.abs(fy[mism] - c) <= NEAR_REL * np.maximum(1.0, np.abs(c))
        assert near.all(), "%s: sign bits differ away from their level" % what
        assert near.sum() <= max(1, MAX_NEAR_FRAC * gs.size), what + ": too many near-level sign flips"
    # S_r depends on every sign; rows with a flipped sign may differ by more
    ok_rows = np.ones(len(rows), bool)
    ok_rows[np.unique(mism[0])] = False
    check_rel(rs[rows][ok_rows], frs[ok_rows], SCALE_RTOL, what + " S_r")


@pytest.mark.parametrize("xdt", ["f32", "f16"])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [16, 32, 128, 256, 4096])
def test_residual_grid(d, bits, xdt):
    n = 444 if d <= 256 else 97
    seed = 31 + d + bits
    say("residual grid d=%d bits=%d x=%s" % (d, bits, xdt))
    x = small_input(n, d, np_dtype(xdt), seed)
    codes, sg, norms, rs = [host(t) for t in rht.residual_quantize(dev(x), bits, seed)]
    check_residual(x, bits, seed, codes, sg, norms, rs)
    assert rs[0] == 0 and norms[0] == 0
    for odt, tol in (("f32", RECON_F32), ("f16", RECON_F16)):
        y = host(rht.residual_dequantize(dev(codes), dev(sg), dev(norms), dev(rs), d, bits, seed,
                                         dtype=tdtype(odt)))
        ref = oracle.residual_dequantize(codes, sg, norms, rs, d, bits, seed, np_dtype(odt))
        check_recon(y, ref, tol, "residual decode %s" % odt)


@pytest.mark.parametrize("xdt", ["f32", "f16"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_residual_extreme_rotated_coordinate(bits, xdt):
    """Rows whose rotation is one-hot: x = D H e_i (entries +-1, exact in fp16), so
    one rotated coordinate reaches the largest possible |y| = sqrt(d) and all others
    are 0; scaled copies, and sums of two such rows."""
    d, seed = 256, 123
    say("residual extreme rotated coordinate bits=%d x=%s" % (bits, xdt))
    s = oracle.signs(seed, d).astype(np.float64)
    idx = np.arange(d)
    rows = []
    for i, scale in ((0, 1.0), (1, 1.0), (77, 0.25), (255, 4.0), (128, 1e-3), (3, 100.0)):
        col = np.where(np.bitwise_count(idx & i) % 2 == 0, 1.0, -1.0)  # H[:, i] (Sylvester)
        rows.append(scale * s * col)
    rows.append(rows[0] + rows[1])
    rows.append(rows[2] - 3 * rows[3])
    x = np.array(rows * 3).astype(np_dtype(xdt))  # 24 rows: several per wave tile
    codes, sg, norms, rs = [host(t) for t in rht.residual_quantize(dev(x), bits, seed)]
    check_residual(x, bits, seed, codes, sg, norms, rs)


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("n", [1, 15, 17, 1000])
def test_residual_decode_arbitrary_inputs(bits, n):
    """The d = 256 decoder on planes no encoder produced: random codes and signs,
    zero norms with a nonzero S_r and the reverse, norms over three decades,
    tiles cut short (n = 1, 15, 17) and several blocks with a tail (n = 1000)."""
    d, seed = 256, 99 + n
    say("residual decode, arbitrary inputs, bits=%d n=%d" % (bits, n))
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(n, d * (bits - 1) // 8), dtype=np.uint8)
    sg = rng.integers(0, 256, size=(n, d // 8), dtype=np.uint8)
    norms = np.exp(rng.uniform(np.log(0.1), np.log(100.0), n)).astype(np.float32)
    rs = (norms * rng.uniform(0.0, 0.3, n)).astype(np.float32)
    norms[::7] = 0.0
    rs[::5] = 0.0
    if n > 1:
        norms[1], rs[1] = 0.0, 0.7  # residual part alone
    for odt, tol in (("f16", RECON_F16), ("f32", RECON_F32)):
        y = host(rht.residual_dequantize(dev(codes), dev(sg), dev(norms), dev(rs), d, bits, seed,
                                         dtype=tdtype(odt)))
        ref = oracle.residual_dequantize(codes, sg, norms, rs, d, bits, seed, np_dtype(odt))
        check_recon(y, ref, tol, "residual decode (arbitrary inputs) %s" % odt)


# ------------------------------------------------------------------ scoring
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("m,n", [(1, 1), (17, 100), (64, 1037), (33, 31), (40, 65), (32, 64)])
def test_score_grid(d, bits, m, n):
    seed = 5 + d
    say("score grid d=%d bits=%d m=%d n=%d" % (d, bits, m, n))
    rng = np.random.default_rng(d * 10 + bits)
    keys = rng.standard_normal((n, d)).astype(np.float32)
    keys[0] = 0.0
    q = rng.standard_normal((m, d)).astype(np.float32)
    codes, norms = oracle.quantize(keys, bits, seed)           # codes from the oracle
    got = host(rht.score(dev(q), dev(codes), dev(norms), d, bits, seed))
    ref = oracle.score(q, codes, norms, d, bits, seed)
    assert np.all(got[:, 0] == 0)
    nz = np.abs(ref).sum(0) > 0
    assert rel_l2(got[:, nz], ref[:, nz]) <= SCORE_TOL
    per_row = rel_l2(got[:, nz], ref[:, nz], axis=1)
    assert per_row.max() <= SCORE_TOL, per_row.max()


@pytest.mark.parametrize("bits", [1, 4])
def test_score_query_scales(bits):
    """Queries spanning 60 decades, a zero query and one whose energy sits in a
    single coordinate: each is scaled into fp16 range by its own power of two."""
    d, n, seed = 128, 300, 77
    say("score query scales bits=%d" % bits)
    rng = np.random.default_rng(bits)
    keys = rng.standard_normal((n, d)).astype(np.float32)
    q = rng.standard_normal((40, d))
    q[0] = 0.0
    q[1] *= 1e-30
    q[2] *= 1e30
    q[3] = 0.0
    q[3, 17] = 3.0
    q[4] *= 1e-3
    q[4, 5] = 1e4
    q[33:] *= np.logspace(-20, 20, 7)[:, None]
    q = q.astype(np.float32)
    codes, norms = oracle.quantize(keys, bits, seed)
    got = host(rht.score(dev(q), dev(codes), dev(norms), d, bits, seed))
    ref = oracle.score(q, codes, norms, d, bits, seed)
    assert np.all(got[0] == 0), "zero query"
    rows = np.arange(1, len(q))
    per_row = rel_l2(got[rows], ref[rows], axis=1)
    assert per_row.max() <= SCORE_TOL, (per_row.max(), rows[per_row.argmax()])


def test_zero_rows_is_a_noop():
    x = torch.zeros((0, 128), dtype=torch.float16, device="cuda:0")
    codes, norms = rht.quantize(x, 4, 1)
    assert codes.shape == (0, 64) and norms.shape == (0,)
    y = rht.dequantize(codes, norms, 128, 4, 1)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


# ------------------------------------------------------------------ workloads
def _mse_workload(w, sample=None, check_all_codes=True):
    """Quantize the whole workload on the GPU; check codes (all rows or a
    sample), norms of all rows, and the decode of a sample of rows."""
    x = testdata.generate(w)
    say("workload %s n=%d d=%d generated" % (w.name, w.n, w.d))
    codes, norms = gpu_quantize(x, w.bits, w.rot_seed)
    _, th, _, _ = oracle.lloyd_max(w.bits)
    rows = np.arange(w.n) if check_all_codes else np.sort(
        np.random.default_rng(w.seed).choice(w.n, size=sample, replace=False))
    parts = chunked(lambda lo, hi: oracle.quantize(x[rows[lo:hi]], w.bits, w.rot_seed), len(rows))
    ocodes = np.concatenate([p[0] for p in parts])
    onorms = np.concatenate([p[1] for p in parts])
    near = check_codes(unpack(codes[rows], w.bits, w.d), unpack(ocodes, w.bits, w.d),
                       lambda r: oracle.quantize(x[rows[r]], w.bits, w.rot_seed, want_y=True)[2], th,
                       w.name + " codes")
    check_rel(norms[rows], onorms, NORM_RTOL, w.name + " norms")
    say("workload %s: %d rows checked, %d near-threshold code mismatches" % (w.name, len(rows), near))
    return x, codes, norms


@pytest.mark.parametrize("odt", ["f32", "f16"])
def test_workload_c1(odt):
    w = testdata.WORKLOADS["c1"]
    x, codes, norms = _mse_workload(w)
    y = host(rht.dequantize(dev(codes), dev(norms), w.d, w.bits, w.rot_seed, dtype=tdtype(odt)))
    ref = oracle.dequantize(codes, norms, w.d, w.bits, w.rot_seed, np_dtype(odt))
    check_recon(y, ref, RECON_F32 if odt == "f32" else RECON_F16, "c1 decode")


@pytest.mark.parametrize("name", ["c2k", "c2v"])
def test_workload_c2_kv_cache(name):
    w = testdata.WORKLOADS[name]
    x, codes, norms = _mse_workload(w, check_all_codes=True)
    del x
    # every row of the decode, on the GPU's own codes
    y = host(rht.dequantize(dev(codes), dev(norms), w.d, w.bits, w.rot_seed, dtype=torch.float16))
    glob, worst = check_recon_all(y, lambda lo, hi: oracle.dequantize(codes[lo:hi], norms[lo:hi], w.d, w.bits,
                                                                      w.rot_seed, np.float16), RECON_F16,
                                  name + " decode")
    say("%s decode, all %d rows: global rel L2 %.2e, worst row %.2e" % (name, w.n, glob, worst))


@pytest.mark.parametrize("mode", [rht.SCALE_SIGN_BIASED, rht.SCALE_SIGN_UNBIASED])
def test_workload_c3_drive(mode):
    w = testdata.WORKLOADS["c3"]
    x = testdata.generate(w)
    say("c3 generated")
    b, S = gpu_quantize(x, 1, w.rot_seed, mode)
    unb = mode == rht.SCALE_SIGN_UNBIASED
    parts = chunked(lambda lo, hi: oracle.sign_quantize(x[lo:hi], unb, w.rot_seed), w.n)
    ob = np.concatenate([p[0] for p in parts])
    oS = np.concatenate([p[1] for p in parts])
    check_codes(unpack(b, 1, w.d), unpack(ob, 1, w.d),
                lambda r: oracle.sign_quantize(x[r], unb, w.rot_seed, want_y=True)[2],
                np.array([0.0]), "c3 bits")
    check_rel(S, oS, SCALE_RTOL, "c3 S")
    y = rht.dequantize(dev(b), dev(S), w.d, 1, w.rot_seed, mode, dtype=torch.float32)
    rows = np.sort(np.random.default_rng(4).choice(w.n, size=4096, replace=False))
    yr = host(y[torch.from_numpy(rows).to("cuda:0")])
    ref = oracle.sign_dequantize(b[rows], S[rows], w.d, w.rot_seed, np.float32)
    check_recon(yr, ref, RECON_F32, "c3 decode")


def test_workload_c4_residual():
    w = testdata.WORKLOADS["c4"]
    x = testdata.generate(w)
    say("c4 generated")
    codes, sg, norms, rs = [host(t) for t in rht.residual_quantize(dev(x), w.bits, w.rot_seed)]
    # every row: stage-1 codes and norms against the oracle's, sign bits and S_r
    # against the oracle run on the GPU's stage-1 codes (row shards in threads)
    chunked(lambda lo, hi: check_residual(x, w.bits, w.rot_seed, codes, sg, norms, rs, rows=np.arange(lo, hi),
                                          what="c4 rows %d-%d" % (lo, hi)), w.n, parts=64)
    say("c4: all %d rows encoded as the oracle encodes them" % w.n)
    for odt, tol in (("f16", RECON_F16), ("f32", RECON_F32)):
        y = host(rht.residual_dequantize(dev(codes), dev(sg), dev(norms), dev(rs), w.d, w.bits, w.rot_seed,
                                         dtype=tdtype(odt)))
        glob, worst = check_recon_all(y, lambda lo, hi: oracle.residual_dequantize(
            codes[lo:hi], sg[lo:hi], norms[lo:hi], rs[lo:hi], w.d, w.bits, w.rot_seed, np_dtype(odt)), tol,
            "c4 decode %s" % odt)
        del y
        say("c4 decode %s, all rows: global rel L2 %.2e, worst row %.2e" % (odt, glob, worst))


def test_workload_c5_scoring():
    wk, wq = testdata.WORKLOADS["c5k"], testdata.WORKLOADS["c5q"]
    keys = testdata.generate(wk)
    q = testdata.generate(wq)
    parts = chunked(lambda lo, hi: oracle.quantize(keys[lo:hi], wk.bits, wk.rot_seed), wk.n)
    codes = np.concatenate([p[0] for p in parts])
    norms = np.concatenate([p[1] for p in parts])
    say("c5 keys quantized by the oracle")
    got = host(rht.score(dev(q), dev(codes), dev(norms), wk.d, wk.bits, wk.rot_seed))
    parts = chunked(lambda lo, hi: oracle.score(q, codes[lo:hi], norms[lo:hi], wk.d, wk.bits,
                                                wk.rot_seed), wk.n)
    ref = np.concatenate(parts, axis=1)
    g = rel_l2(got, ref)
    per_row = rel_l2(got, ref, axis=1)
    say("c5 score: global rel L2 %.2e, worst query %.2e" % (g, per_row.max()))
    assert g <= SCORE_TOL and per_row.max() <= SCORE_TOL
