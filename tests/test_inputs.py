"""The seeded input generators (testdata/) on the CPU: every row is a function of
its index alone (any slice, any thread count, any order gives the same bytes),
and each workload has the distribution its recipe states: N(0,1) coordinates,
the named outlier channels scaled by their factor, per-row log-normal scales,
Student-t (nu = 3) coordinates for the DRIVE workload."""
import numpy as np
import pytest
from scipy import stats

from testdata import WORKLOADS, generate, generate_rows, scaled


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_rows_depend_on_their_index_only(name):
    w = scaled(WORKLOADS[name], 300)
    full = generate(w, nthreads=1)
    assert full.dtype == w.np_dtype and full.shape == (300, w.d)
    np.testing.assert_array_equal(generate(w, nthreads=4), full)
    np.testing.assert_array_equal(generate(w, row0=100, nrows=57, nthreads=3), full[100:157])
    rows = np.array([299, 0, 150, 150, 7])
    np.testing.assert_array_equal(generate_rows(w, rows), full[rows])
    # a longer workload of the same recipe starts with the same rows
    np.testing.assert_array_equal(generate(scaled(w, 400), nrows=300), full)
    assert np.all(np.isfinite(full.astype(np.float64)))


def test_seeds_give_different_data():
    a = generate(scaled(WORKLOADS["c2k"], 64))
    b = generate(scaled(WORKLOADS["c2v"], 64))
    assert np.mean(a == b) < 0.01


def channel_std(x):
    return x.astype(np.float64).std(axis=0)


def rest(w, x):
    keep = np.ones(w.d, bool)
    keep[w.outlier_channels()] = False
    return x.astype(np.float64)[:, keep]


def test_c1_gaussian_with_two_fixed_outlier_channels():
    w = WORKLOADS["c1"]
    x = generate(w)
    assert list(w.outlier_channels()) == [3, 77]
    s = channel_std(x)
    np.testing.assert_allclose(s[[3, 77]], 20.0, rtol=0.05)
    r = rest(w, x)
    assert abs(r.mean()) < 0.01 and abs(r.std() - 1.0) < 0.01


@pytest.mark.parametrize("name,count,mult", [("c2k", 1, 20.0), ("c2v", 1, 20.0), ("c4", 5, 30.0)])
def test_seeded_outlier_channels(name, count, mult):
    w = scaled(WORKLOADS[name], 20000)
    ch = w.outlier_channels()
    assert len(ch) == count == len(set(ch.tolist())) and ch.min() >= 0 and ch.max() < w.d
    x = generate(w)
    s = channel_std(x)
    base = np.median(np.delete(s, ch))
    np.testing.assert_allclose(s[ch] / base, mult, rtol=0.05)


@pytest.mark.parametrize("name", ["c2k", "c2v"])
def test_kv_rows_have_log_normal_scales(name):
    """Each row is an N(0,1) vector (plus its outlier channel) times exp(0.5 g):
    the log of a row's rms over the ordinary channels has sd 0.5 and mean 0, up to
    the small spread of the rms of 127 normals (~1/sqrt(254))."""
    w = scaled(WORKLOADS[name], 20000)
    r = rest(w, generate(w))
    lr = np.log(np.sqrt((r ** 2).mean(axis=1)))
    assert abs(lr.std() - np.sqrt(0.25 + 1.0 / 254)) < 0.015
    assert abs(lr.mean()) < 0.015


def test_c3_student_t_three_degrees():
    w = scaled(WORKLOADS["c3"], 2048)
    x = generate(w).astype(np.float64).ravel()
    tail = np.mean(np.abs(x) > 5.0)
    np.testing.assert_allclose(tail, 2 * stats.t.sf(5.0, 3), rtol=0.05)
    np.testing.assert_allclose(np.median(np.abs(x)), stats.t.ppf(0.75, 3), rtol=0.01)
    # the whole distribution, by a Kolmogorov-Smirnov distance on a sample
    assert stats.kstest(x[::37], stats.t(3).cdf).statistic < 0.01


@pytest.mark.parametrize("name", ["c5k", "c5q"])
def test_scoring_inputs_are_standard_normal(name):
    w = WORKLOADS[name]
    x = generate(scaled(w, min(w.n, 8192))).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.02
    assert stats.kstest(x.ravel()[::7], "norm").pvalue > 1e-3
