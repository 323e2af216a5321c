"""The attention tolerance (parity.attention_bound) is checked on the CPU
against an emulation of the kernel's arithmetic in numpy: fp16 hi + lo parts
of the rotated query, of the codebook levels and of the softmax weights,
products and sums in fp32.  The faithful emulation must stay inside the bound;
the same emulation with the query's lo part dropped (an error of about 2^-11
per product) must leave it, so the bound separates fp32-level rounding from a
lost term.  No GPU is used; the reference is the oracle's plain definition.
"""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle
from parity import attention_bound, attention_terms

D, BITS = 128, 4
LOG2E = 1.4426950408889634


def split(x):
    hi = x.astype(np.float16).astype(np.float32)
    lo = (x - hi).astype(np.float16).astype(np.float32)
    return hi, lo


def emulate(q, kc, kn, vc, vn, sk, sv, scale, drop_query_lo=False, value_scale="weight"):
    """value_scale: the power of two that brings the value weights p ||v|| into
    fp16 range comes from the largest weight ("weight", as the kernel does) or
    from the largest norm alone ("norm", which loses the weights of ordinary
    keys when a negligible one has a huge norm)."""
    lv = oracle.lloyd_max(BITS)[0].astype(np.float32)
    ch, cl = split(lv)
    Hm = scipy.linalg.hadamard(D).astype(np.float64)
    dk = oracle.signs(sk, D).astype(np.float64)
    dv = oracle.signs(sv, D).astype(np.float64)
    heads, m, _ = q.shape
    out = np.zeros((heads, m, D), np.float32)
    for h in range(heads):
        kcode = np.stack([kc[h] & 15, kc[h] >> 4], -1).reshape(kc.shape[1], D)
        vcode = np.stack([vc[h] & 15, vc[h] >> 4], -1).reshape(vc.shape[1], D)
        for i in range(m):
            qt = (Hm @ (dk * q[h, i].astype(np.float64))).astype(np.float32)
            mx = np.abs(qt).max()
            sq = np.float32(2.0 ** (14 - math.frexp(float(mx))[1])) if mx > 0 else np.float32(1)
            qh, ql = split(qt * sq)
            if drop_query_lo:
                ql = np.zeros_like(ql)
            c = ((ch[kcode] * qh).sum(1, dtype=np.float32) + (cl[kcode] * qh).sum(1, dtype=np.float32)
                 + (ch[kcode] * ql).sum(1, dtype=np.float32))
            fq = np.float32(scale * LOG2E / (D * sq))
            s = c * kn[h] * fq
            p = np.exp2(s - s.max()).astype(np.float32)
            wmax = (p * vn[h]).max() if value_scale == "weight" else vn[h].max()
            vs = np.float32(2.0 ** (14 - math.frexp(float(wmax))[1])) if wmax > 0 else np.float32(1)
            P = p * vn[h] * vs
            ph, pl = split(P)
            z = ((ph[:, None] * ch[vcode]).sum(0, dtype=np.float32) + (pl[:, None] * ch[vcode]).sum(0, dtype=np.float32)
                 + (ph[:, None] * cl[vcode]).sum(0, dtype=np.float32))
            z = z / np.float32(vs * D) / p.sum(dtype=np.float32)
            out[h, i] = (dv * (Hm @ z.astype(np.float64))).astype(np.float32)
    return out


def decoded(codes, norms, seed):
    heads, n, _ = codes.shape
    y = oracle.dequantize(codes.reshape(heads * n, -1), norms.reshape(-1), D, BITS, seed, np.float32)
    return y.reshape(heads, n, D).astype(np.float64)


@pytest.mark.parametrize("scale,qmul", [(1 / math.sqrt(D), 1.0), (1.0, 2.0), (1 / math.sqrt(D), 30.0)])
def test_bound_separates_rounding_from_a_lost_term(scale, qmul):
    rng = np.random.default_rng(int(qmul * 10))
    heads, m, n = 2, 4, 500
    x = rng.standard_normal((2 * heads * n, D)).astype(np.float32)
    kc, kn = oracle.quantize(x[: heads * n], BITS, 81)
    vc, vn = oracle.quantize(x[heads * n:], BITS, 82)
    kc, vc = kc.reshape(heads, n, -1), vc.reshape(heads, n, -1)
    kn, vn = kn.reshape(heads, n), vn.reshape(heads, n)
    q = (qmul * rng.standard_normal((heads, m, D))).astype(np.float32)
    ref = oracle.attention(q, kc, kn, vc, vn, D, BITS, BITS, 81, 82, scale)
    qt, kterm = attention_terms(q, kc, kn, D, BITS, 81, oracle.lloyd_max(BITS)[0],
                                oracle.signs(81, D).astype(np.float64), scipy.linalg.hadamard(D))
    bound = attention_bound(q, qt, kterm, decoded(kc, kn, 81), decoded(vc, vn, 82), ref, scale)
    good = np.linalg.norm(emulate(q, kc, kn, vc, vn, 81, 82, scale) - ref, axis=2)
    bad = np.linalg.norm(emulate(q, kc, kn, vc, vn, 81, 82, scale, drop_query_lo=True) - ref, axis=2)
    assert np.all(good <= bound), (good / bound).max()
    # a lost term shows wherever the output depends on the logits at all
    assert (bad / bound).max() > 10, (bad / bound).max()
    assert (good / bound).max() < 0.25, (good / bound).max()


def test_value_scale_follows_the_weights():
    # value norms over 40 decades and near-hard attention: the key that wins the
    # softmax has an ordinary norm while keys of negligible weight reach 1e20
    rng = np.random.default_rng(7)
    heads, m, n = 2, 3, 300
    x = rng.standard_normal((2 * heads * n, D)).astype(np.float32)
    x[heads * n:] *= (10.0 ** rng.uniform(-20, 20, heads * n)).astype(np.float32)[:, None]
    kc, kn = oracle.quantize(x[: heads * n], BITS, 91)
    vc, vn = oracle.quantize(x[heads * n:], BITS, 92)
    kc, vc = kc.reshape(heads, n, -1), vc.reshape(heads, n, -1)
    kn, vn = kn.reshape(heads, n), vn.reshape(heads, n)
    q = rng.standard_normal((heads, m, D)).astype(np.float32)
    q[:, 1] *= 1e4
    scale = 1 / math.sqrt(D)
    ref = oracle.attention(q, kc, kn, vc, vn, D, BITS, BITS, 91, 92, scale)
    qt, kterm = attention_terms(q, kc, kn, D, BITS, 91, oracle.lloyd_max(BITS)[0],
                                oracle.signs(91, D).astype(np.float64), scipy.linalg.hadamard(D))
    bound = attention_bound(q, qt, kterm, decoded(kc, kn, 91), decoded(vc, vn, 92), ref, scale)
    good = np.linalg.norm(emulate(q, kc, kn, vc, vn, 91, 92, scale) - ref, axis=2)
    bad = np.linalg.norm(emulate(q, kc, kn, vc, vn, 91, 92, scale, value_scale="norm") - ref, axis=2)
    assert np.all(good <= bound), (good / bound).max()
    assert (bad / bound).max() > 10, (bad / bound).max()
