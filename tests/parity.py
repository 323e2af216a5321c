"""Comparison rules shared by the GPU parity tests (GPU result vs CPU oracle).

* Codes / sign bits: bit-exact, except that a coordinate may differ by exactly
  one level when the oracle's fp64 normalized value y lies within 1e-5 *
  max(1, |t|) of the decision threshold t between the two codes.  Such
  near-threshold mismatches are counted and must stay below 1e-6 of all codes
  (at least one is tolerated when 1e-6 of the count is below one code).
* Norms: relative 1e-6.  Scales S, S_r: relative 1e-5.
* Reconstructions and scores are compared on identical code bytes (the oracle
  decodes the GPU's codes), per row and globally, relative L2 <= 1e-5 for fp32
  outputs and 2e-3 for fp16 outputs.
* Attention outputs: the error model of attention_bound (fp16 hi/lo operands,
  fp32 sums), per (head, query) row.
"""
from __future__ import annotations

import concurrent.futures
import math
import os

import numpy as np

NEAR_REL = 1e-5
MAX_NEAR_FRAC = 1e-6
NORM_RTOL = 1e-6
SCALE_RTOL = 1e-5
RECON_F32 = 1e-5
RECON_F16 = 2e-3
SCORE_TOL = 1e-5
# Attention error model.  The kernel forms every product from fp16 hi + lo
# parts (x = hi + lo to 2^-22 relative) and sums them in fp32.  Per key j:
#   products:   each logit s_j is a sum of d products t_jk.  Every product
#               misses lo*lo and the rounding of the two lo parts, each at most
#               2^-22 |t_jk|; the fp32 sums add a few 2^-24 of the sum's size.
#               The query's and the 16 codebook levels' splits are fixed, but
#               key j meets them through its own codes, so across keys these
#               errors behave like independent ones: a logit is off by about
#               ATTN_GAMMA_R * T_j, T_j = ||(t_jk)_k||_2, and the errors of
#               different keys add in quadrature.  The value products carry
#               the same relative error;
#   final:      normalization, merging of chunks and the inverse transform,
#               ATTN_GAMMA_F relative to the output.
# A logit error ds_j moves the output by sum_j p_j ds_j (v_j - out).  Per (head, query):
#   ||gpu - ref|| <= ATTN_SAFETY * [ ATTN_GAMMA_R sqrt(sum_j p_j^2 (T_j^2 ||v_j - ref||^2 + ||v_j||^2))
#                    + ATTN_GAMMA_F ||ref|| ]
# with ATTN_SAFETY a six-sigma margin on these rms estimates.
ATTN_GAMMA_R = 2 * 2.0 ** -22 + 4 * 2.0 ** -24
ATTN_GAMMA_F = 8 * 2.0 ** -24
ATTN_SAFETY = 6.0


def unpack(codes: np.ndarray, width: int, d: int) -> np.ndarray:
    bits = np.unpackbits(np.ascontiguousarray(codes), axis=-1, bitorder="little")[..., : width * d]
    bits = bits.reshape(*codes.shape[:-1], d, width).astype(np.int16)
    return (bits << np.arange(width, dtype=np.int16)).sum(-1).astype(np.int16)


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def chunked(fn, n: int, parts: int | None = None):
    """Run fn(lo, hi) over row ranges in threads (the oracle releases the GIL)."""
    parts = parts or threads()
    edges = np.linspace(0, n, parts + 1).astype(np.int64)
    with concurrent.futures.ThreadPoolExecutor(min(parts, threads())) as ex:
        return list(ex.map(lambda i: fn(int(edges[i]), int(edges[i + 1])), range(parts)))


def check_codes(gpu: np.ndarray, ref: np.ndarray, y_of_rows, thresholds: np.ndarray,
                what: str) -> int:
    """gpu/ref: unpacked int codes [n][d].  y_of_rows(rows) -> fp64 y for those
    rows.  thresholds[k] separates code k and k+1.  Returns the number of
    near-threshold mismatches; raises on any other mismatch."""
    diff = gpu != ref
    nmis = int(diff.sum())
    if nmis == 0:
        return 0
    rows = np.unique(np.nonzero(diff)[0])
    y = y_of_rows(rows)
    g, r = gpu[rows], ref[rows]
    bad = []
    near = 0
    for i, j in zip(*np.nonzero(g != r)):
        lo = min(int(g[i, j]), int(r[i, j]))
        if abs(int(g[i, j]) - int(r[i, j])) != 1:
            bad.append((rows[i], j, int(g[i, j]), int(r[i, j]), y[i, j]))
            continue
        t = float(thresholds[lo])
        if abs(y[i, j] - t) <= NEAR_REL * max(1.0, abs(t)):
            near += 1
        else:
            bad.append((rows[i], j, int(g[i, j]), int(r[i, j]), y[i, j]))
    assert not bad, "%s: %d code mismatches away from a threshold, e.g. %s" % (what, len(bad), bad[:5])
    total = gpu.size
    assert near <= max(1, MAX_NEAR_FRAC * total), \
        "%s: %d near-threshold mismatches in %d codes" % (what, near, total)
    return near


def rel_l2(a: np.ndarray, b: np.ndarray, axis=None):
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    num = np.sqrt(((a - b) ** 2).sum(axis=axis))
    den = np.sqrt((b ** 2).sum(axis=axis))
    return num / np.maximum(den, 1e-300)


def check_recon(gpu: np.ndarray, ref: np.ndarray, tol: float, what: str):
    ref64 = ref.astype(np.float64)
    nz = (ref64 ** 2).sum(1) > 0
    per_row = rel_l2(gpu[nz], ref[nz], axis=1)
    glob = rel_l2(gpu, ref)
    assert per_row.size == 0 or per_row.max() <= tol, \
        "%s: worst row rel L2 %.3g > %.1g (row %d)" % (what, per_row.max(), tol,
                                                     np.nonzero(nz)[0][per_row.argmax()])
    assert glob <= tol, "%s: global rel L2 %.3g > %.1g" % (what, glob, tol)
    # rows whose reference is exactly zero must decode to exactly zero
    assert np.all(gpu[~nz] == 0), "%s: zero rows not decoded to zero" % what
    return float(glob), float(per_row.max()) if per_row.size else 0.0


def check_recon_all(gpu: np.ndarray, ref_rows, tol: float, what: str, rows_per_part: int = 1 << 16):
    """check_recon over every row of a large output without a second full copy:
    ref_rows(lo, hi) -> the oracle's rows [lo, hi); parts run in threads (the
    oracle releases the GIL).  Same rules: per-row and global relative L2 <= tol,
    zero reference rows decode to exactly zero.  Returns (global, worst row)."""
    n = gpu.shape[0]
    edges = list(range(0, n, rows_per_part)) + [n]

    def part(i):
        lo, hi = edges[i], edges[i + 1]
        ref = ref_rows(lo, hi).astype(np.float64)
        g = gpu[lo:hi].astype(np.float64)
        den = (ref ** 2).sum(1)
        num = ((g - ref) ** 2).sum(1)
        nz = den > 0
        worst = float(np.sqrt(num[nz] / den[nz]).max()) if nz.any() else 0.0
        zero_ok = bool(np.all(g[~nz] == 0))
        return float(num.sum()), float(den.sum()), worst, zero_ok, lo + (int(np.argmax(np.where(nz, num / np.maximum(den, 1e-300), 0))) if nz.any() else 0)

    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, range(len(edges) - 1)))
    num = sum(r[0] for r in res)
    den = sum(r[1] for r in res)
    worst = max(r[2] for r in res)
    at = max(res, key=lambda r: r[2])[4]
    assert all(r[3] for r in res), "%s: zero rows not decoded to zero" % what
    assert worst <= tol, "%s: worst row rel L2 %.3g > %.1g (row %d)" % (what, worst, tol, at)
    glob = math.sqrt(num / max(den, 1e-300))
    assert glob <= tol, "%s: global rel L2 %.3g > %.1g" % (what, glob, tol)
    return glob, worst


def check_rel(gpu: np.ndarray, ref: np.ndarray, rtol: float, what: str):
    gpu = gpu.astype(np.float64)
    ref = ref.astype(np.float64)
    err = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-30)
    err[(ref == 0) & (gpu == 0)] = 0
    assert err.max() <= rtol, "%s: max rel err %.3g > %.1g at %d (gpu %r ref %r)" % (
        what, err.max(), rtol, err.argmax(), gpu.flat[err.argmax()], ref.flat[err.argmax()])
    return float(err.max())


def attention_bound(q, qt, kterm, kd, vd, ref, scale):
    """Per (head, query) bound on ||gpu - ref|| from the error model above.
    q [heads][m][d] queries; qt [heads][m][d] their rotations H D_k q; kterm
    [heads][n][d] the factors (||k_j|| / d) c[code_jk] with which the rotated
    query meets key j; kd, vd [heads][n][d] decoded keys and values; ref the
    oracle output [heads][m][d]."""
    out = np.zeros(ref.shape[:2])
    for h in range(q.shape[0]):
        s = scale * (q[h].astype(np.float64) @ kd[h].T)                          # [m][n]
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        T = abs(scale) * np.sqrt((qt[h] ** 2) @ (kterm[h] ** 2).T)               # [m][n]
        vnorm2 = (vd[h] ** 2).sum(1)                                             # [n]
        spread2 = ((vd[h][None, :, :] - ref[h][:, None, :]) ** 2).sum(2)         # [m][n]
        rand = np.sqrt((p ** 2 * (T ** 2 * spread2 + vnorm2[None, :])).sum(1))
        out[h] = ATTN_SAFETY * (ATTN_GAMMA_R * rand + ATTN_GAMMA_F * np.linalg.norm(ref[h], axis=1))
    return out


def attention_terms(q, kc, kn, d, bits, seed_k, levels, signs_k, hadamard):
    """Inputs of attention_bound: the rotated queries H D_k q and the factors
    (||k_j|| / d) c[code_jk], from the oracle's codebook and signs and a dense
    Hadamard matrix."""
    qt = np.einsum("ij,hmj->hmi", hadamard, q.astype(np.float64) * signs_k[None, None, :])
    code = unpack(kc.reshape(-1, kc.shape[-1]), bits, d).reshape(kc.shape[0], kc.shape[1], d)
    kterm = levels[code] * (kn.astype(np.float64) / d)[..., None]
    return qt, kterm
