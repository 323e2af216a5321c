"""CPU oracle for random-rotation (randomized Hadamard) vector quantization.

TEST INFRASTRUCTURE. This package is the plain, slow, fp64 reference that the
HIP library is checked against. Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
does, and it imports nothing from the product package.

The arithmetic lives in ``rht_oracle.c`` (plain C99, single-threaded); this
module only compiles it with gcc and marshals numpy arrays through ctypes.
Every function cites the passage of the web page "Random-rotation
quantization" it follows; see the header of ``rht_oracle.c`` for the
citation keys and for the readings taken where the page is silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rht_oracle.c")
_LIB = os.path.join(_HERE, "librho.so")

F32 = 0
F16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, ISO C99 so no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
        L.rho_abi.restype = i32
        L.rho_splitmix64_next.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
        L.rho_splitmix64_next.restype = ctypes.c_uint64
        L.rho_signs.argtypes = [u64, i32, vp]
        L.rho_fwht.argtypes = [vp, i32]
        L.rho_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.rho_f16_to_f64.restype = ctypes.c_double
        L.rho_f64_to_f16.argtypes = [ctypes.c_double]
        L.rho_f64_to_f16.restype = ctypes.c_uint16
        L.rho_lloyd_max.argtypes = [i32, vp, vp, vp, vp]
        L.rho_quantize.argtypes = [vp, i32, i64, i32, i32, u64, vp, vp, vp]
        L.rho_quantize_eden.argtypes = [vp, i32, i64, i32, i32, u64, vp, vp]
        L.rho_lloyd_max_beta.argtypes = [i32, i32, vp, vp, vp, vp]
        L.rho_quantize_cb.argtypes = [vp, i32, i64, i32, i32, u64, vp, vp, vp, vp, vp]
        L.rho_dequantize_cb.argtypes = [vp, vp, i64, i32, i32, u64, vp, vp, i32]
        L.rho_score_sign.argtypes = [vp, i32, vp, vp, i64, i32, u64, vp]
        L.rho_score_sign_dense.argtypes = [vp, i32, vp, vp, i64, i32, u64, vp]
        L.rho_score_residual.argtypes = [vp, i32, vp, vp, vp, vp, i64, i32, i32, u64, vp]
        L.rho_score_residual_dense.argtypes = [vp, i32, vp, vp, vp, vp, i64, i32, i32, u64, vp]
        for f in (L.rho_attention, L.rho_attention_rotated):
            f.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i32, i32, i32, u64, u64, ctypes.c_double, vp]
        L.rho_dequantize.argtypes = [vp, vp, i64, i32, i32, u64, vp, i32]
        L.rho_sign_quantize.argtypes = [vp, i32, i64, i32, i32, u64, vp, vp, vp]
        L.rho_sign_dequantize.argtypes = [vp, vp, i64, i32, u64, vp, i32]
        L.rho_residual_quantize.argtypes = [vp, i32, i64, i32, i32, u64, vp, vp, vp, vp, vp, vp]
        L.rho_residual_dequantize.argtypes = [vp, vp, vp, vp, i64, i32, i32, u64, vp, i32]
        L.rho_score.argtypes = [vp, i32, vp, vp, i64, i32, i32, u64, vp]
        L.rho_score_dense.argtypes = [vp, i32, vp, vp, i64, i32, i32, u64, vp]
        for name in ("rho_lloyd_max", "rho_quantize", "rho_dequantize", "rho_sign_quantize",
                     "rho_sign_dequantize", "rho_residual_quantize", "rho_residual_dequantize",
                     "rho_score", "rho_score_dense"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.float16:
        return F16
    raise TypeError("oracle inputs are float32 or float16, got %s" % x.dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def _np_out_dtype(code: int):
    return np.float16 if code == F16 else np.float32


# --------------------------------------------------------------------------
def splitmix64_stream(seed: int, count: int) -> list[int]:
    """The first `count` SplitMix64 outputs from state `seed`."""
    st = ctypes.c_uint64(seed)
    return [int(lib().rho_splitmix64_next(ctypes.byref(st))) for _ in range(count)]


def signs(seed: int, d: int) -> np.ndarray:
    """Diagonal D of the randomized Hadamard transform: int8 +-1 of length d."""
    s = np.empty(d, dtype=np.int8)
    lib().rho_signs(seed, d, _p(s))
    return s


def fwht(v: np.ndarray) -> np.ndarray:
    """Unnormalized Sylvester-order fast Walsh-Hadamard transform of each row."""
    a = np.array(v, dtype=np.float64, copy=True, order="C")
    d = a.shape[-1]
    flat = a.reshape(-1, d)
    for r in range(flat.shape[0]):
        row = flat[r]
        lib().rho_fwht(row.ctypes.data_as(ctypes.c_void_p), d)
    return a


def f16_to_f64(bits: int) -> float:
    return float(lib().rho_f16_to_f64(bits))


def f64_to_f16(v: float) -> int:
    return int(lib().rho_f64_to_f16(v))


def lloyd_max(bits: int):
    """(levels[2^b], thresholds[2^b - 1], mse, iterations) for N(0,1)."""
    K = 1 << bits
    lv = np.zeros(K, np.float64)
    th = np.zeros(max(K - 1, 1), np.float64)
    mse = np.zeros(1, np.float64)
    it = np.zeros(1, np.int32)
    _check(lib().rho_lloyd_max(bits, _p(lv), _p(th), _p(mse), _p(it)), "lloyd_max")
    return lv, th[: K - 1], float(mse[0]), int(it[0])


def lloyd_max_beta(bits: int, d: int):
    """(levels, thresholds, mse, iterations) of the Lloyd-Max codebook for the
    exact marginal of sqrt(d) * (a coordinate of a uniformly rotated unit vector)."""
    K = 1 << bits
    lv = np.zeros(K, np.float64)
    th = np.zeros(max(K - 1, 1), np.float64)
    mse = np.zeros(1, np.float64)
    it = np.zeros(1, np.int32)
    _check(lib().rho_lloyd_max_beta(bits, d, _p(lv), _p(th), _p(mse), _p(it)), "lloyd_max_beta")
    return lv, th[: K - 1], float(mse[0]), int(it[0])


def quantize_cb(x: np.ndarray, bits: int, seed: int, levels, thresholds, want_y: bool = False):
    """MSE encoder with the given codebook: (codes, norms[, y])."""
    x = np.ascontiguousarray(x)
    n, d = x.shape
    lv = np.ascontiguousarray(levels, dtype=np.float64)
    th = np.ascontiguousarray(thresholds, dtype=np.float64)
    codes = np.zeros((n, bits * d // 8), np.uint8)
    norms = np.zeros(n, np.float32)
    y = np.zeros((n, d), np.float64) if want_y else None
    _check(lib().rho_quantize_cb(_p(x), _dtype_code(x), n, d, bits, seed, _p(lv), _p(th), _p(codes), _p(norms),
                                 _p(y)), "quantize_cb")
    return (codes, norms, y) if want_y else (codes, norms)


def dequantize_cb(codes, norms, d: int, bits: int, seed: int, levels, out_dtype=np.float32):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    lv = np.ascontiguousarray(levels, dtype=np.float64)
    n = norms.shape[0]
    oc = F16 if np.dtype(out_dtype) == np.float16 else F32
    out = np.zeros((n, d), _np_out_dtype(oc))
    _check(lib().rho_dequantize_cb(_p(codes), _p(norms), n, d, bits, seed, _p(lv), _p(out), oc), "dequantize_cb")
    return out


def quantize(x: np.ndarray, bits: int, seed: int, want_y: bool = False):
    """MSE encoder: returns (codes u8[n][bits*d/8], norms f32[n][, y f64[n][d]])."""
    x = np.ascontiguousarray(x)
    n, d = x.shape
    codes = np.zeros((n, bits * d // 8), np.uint8)
    norms = np.zeros(n, np.float32)
    y = np.zeros((n, d), np.float64) if want_y else None
    _check(lib().rho_quantize(_p(x), _dtype_code(x), n, d, bits, seed, _p(codes), _p(norms), _p(y)),
           "quantize")
    return (codes, norms, y) if want_y else (codes, norms)


def quantize_eden(x: np.ndarray, bits: int, seed: int):
    """MSE codes with the EDEN-style unbiased scale S = d ||x||^2 / <c, H D x>:
    (codes u8[n][bits*d/8], S f32[n]); decode with dequantize()."""
    x = np.ascontiguousarray(x)
    n, d = x.shape
    codes = np.zeros((n, bits * d // 8), np.uint8)
    S = np.zeros(n, np.float32)
    _check(lib().rho_quantize_eden(_p(x), _dtype_code(x), n, d, bits, seed, _p(codes), _p(S)), "quantize_eden")
    return codes, S


def dequantize(codes: np.ndarray, norms: np.ndarray, d: int, bits: int, seed: int,
               out_dtype=np.float32) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    n = norms.shape[0]
    oc = F16 if np.dtype(out_dtype) == np.float16 else F32
    out = np.zeros((n, d), _np_out_dtype(oc))
    _check(lib().rho_dequantize(_p(codes), _p(norms), n, d, bits, seed, _p(out), oc), "dequantize")
    return out


def sign_quantize(x: np.ndarray, unbiased: bool, seed: int, want_y: bool = False):
    """DRIVE 1-bit encoder: (bits u8[n][d/8], S f32[n][, y])."""
    x = np.ascontiguousarray(x)
    n, d = x.shape
    b = np.zeros((n, d // 8), np.uint8)
    S = np.zeros(n, np.float32)
    y = np.zeros((n, d), np.float64) if want_y else None
    _check(lib().rho_sign_quantize(_p(x), _dtype_code(x), n, d, int(bool(unbiased)), seed, _p(b),
                                   _p(S), _p(y)), "sign_quantize")
    return (b, S, y) if want_y else (b, S)


def sign_dequantize(bits: np.ndarray, S: np.ndarray, d: int, seed: int, out_dtype=np.float32):
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    S = np.ascontiguousarray(S, dtype=np.float32)
    n = S.shape[0]
    oc = F16 if np.dtype(out_dtype) == np.float16 else F32
    out = np.zeros((n, d), _np_out_dtype(oc))
    _check(lib().rho_sign_dequantize(_p(bits), _p(S), n, d, seed, _p(out), oc), "sign_dequantize")
    return out


def residual_quantize(x: np.ndarray, bits: int, seed: int, forced_codes=None, want_y=False):
    """Residual chain: (codes[n][(b-1)d/8], signs[n][d/8], norms, res_scale[, y])."""
    x = np.ascontiguousarray(x)
    n, d = x.shape
    codes = np.zeros((n, (bits - 1) * d // 8), np.uint8)
    sg = np.zeros((n, d // 8), np.uint8)
    norms = np.zeros(n, np.float32)
    rs = np.zeros(n, np.float32)
    y = np.zeros((n, d), np.float64) if want_y else None
    fc = None if forced_codes is None else np.ascontiguousarray(forced_codes, dtype=np.uint8)
    _check(lib().rho_residual_quantize(_p(x), _dtype_code(x), n, d, bits, seed, _p(fc), _p(codes),
                                       _p(sg), _p(norms), _p(rs), _p(y)), "residual_quantize")
    out = (codes, sg, norms, rs)
    return out + (y,) if want_y else out


def residual_dequantize(codes, sg, norms, rs, d: int, bits: int, seed: int, out_dtype=np.float32):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sg = np.ascontiguousarray(sg, dtype=np.uint8)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    rs = np.ascontiguousarray(rs, dtype=np.float32)
    n = norms.shape[0]
    oc = F16 if np.dtype(out_dtype) == np.float16 else F32
    out = np.zeros((n, d), _np_out_dtype(oc))
    _check(lib().rho_residual_dequantize(_p(codes), _p(sg), _p(norms), _p(rs), n, d, bits, seed,
                                         _p(out), oc), "residual_dequantize")
    return out


def score(q: np.ndarray, codes: np.ndarray, norms: np.ndarray, d: int, bits: int, seed: int):
    """Rotated-domain scoring on the codes: fp32 logits[m][n]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    m, n = q.shape[0], norms.shape[0]
    out = np.zeros((m, n), np.float32)
    _check(lib().rho_score(_p(q), m, _p(codes), _p(norms), n, d, bits, seed, _p(out)), "score")
    return out


def score_dense(q: np.ndarray, codes: np.ndarray, norms: np.ndarray, d: int, bits: int, seed: int):
    """The plain definition: fp64 Q . dequant(K)^T."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    m, n = q.shape[0], norms.shape[0]
    out = np.zeros((m, n), np.float64)
    _check(lib().rho_score_dense(_p(q), m, _p(codes), _p(norms), n, d, bits, seed, _p(out)),
           "score_dense")
    return out


def _attention(fn, name, q, kc, kn, vc, vn, d, k_bits, v_bits, seed_k, seed_v, scale):
    q = np.ascontiguousarray(q, dtype=np.float32)
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    kn = np.ascontiguousarray(kn, dtype=np.float32)
    vn = np.ascontiguousarray(vn, dtype=np.float32)
    heads, m = q.shape[0], q.shape[1]
    n = kn.shape[1]
    assert q.shape == (heads, m, d) and kn.shape == (heads, n) and vn.shape == (heads, n)
    assert kc.shape == (heads, n, k_bits * d // 8) and vc.shape == (heads, n, v_bits * d // 8)
    out = np.zeros((heads, m, d), np.float64)
    _check(fn(_p(q), m, _p(kc), _p(kn), _p(vc), _p(vn), heads, n, d, k_bits, v_bits, seed_k, seed_v,
              float(scale), _p(out)), name)
    return out


def attention(q, kc, kn, vc, vn, d, k_bits, v_bits, seed_k, seed_v, scale):
    """Attention over coded keys and values, plain definition (fp64):
    softmax(scale * q . dequant(K)^T) . dequant(V) per head, keys decoded with
    the k_bits codebook, values with the v_bits one.
    q [heads][m][d], codes [heads][n][bits*d/8], norms [heads][n]."""
    return _attention(lib().rho_attention, "attention", q, kc, kn, vc, vn, d, k_bits, v_bits, seed_k,
                      seed_v, scale)


def attention_rotated(q, kc, kn, vc, vn, d, k_bits, v_bits, seed_k, seed_v, scale):
    """The same attention in the rotated domains: logits on the codes, value
    sum kept rotated, one inverse transform per query (fp64)."""
    return _attention(lib().rho_attention_rotated, "attention_rotated", q, kc, kn, vc, vn, d, k_bits,
                      v_bits, seed_k, seed_v, scale)


def score_sign(q, bits, scale, d: int, seed: int, dense: bool = False):
    """<q, x^> for sign-coded keys (either DRIVE scale): fp32 logits[m][n] on
    the codes, or with dense=True the fp64 plain definition."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    m, n = q.shape[0], scale.shape[0]
    out = np.zeros((m, n), np.float64 if dense else np.float32)
    fn = lib().rho_score_sign_dense if dense else lib().rho_score_sign
    _check(fn(_p(q), m, _p(bits), _p(scale), n, d, seed, _p(out)), "score_sign")
    return out


def score_residual(q, codes, signs, norms, res_scale, d: int, bits: int, seed: int, dense: bool = False):
    """<q, x^> for residual-chain-coded keys: fp32 logits[m][n] on the codes,
    or with dense=True the fp64 plain definition."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    signs = np.ascontiguousarray(signs, dtype=np.uint8)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    res_scale = np.ascontiguousarray(res_scale, dtype=np.float32)
    m, n = q.shape[0], norms.shape[0]
    out = np.zeros((m, n), np.float64 if dense else np.float32)
    fn = lib().rho_score_residual_dense if dense else lib().rho_score_residual
    _check(fn(_p(q), m, _p(codes), _p(signs), _p(norms), _p(res_scale), n, d, bits, seed, _p(out)),
           "score_residual")
    return out
