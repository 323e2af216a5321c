"""Python binding of librht: randomized-Hadamard vector quantization on MI355X.

The heavy lifting is in ``librht.so`` (hand-written HIP kernels for gfx950
behind the C ABI declared in ``include/rht.h``).  This module only marshals
arguments:

* ``rht_quantize`` ... ``rht_signs`` mirror the C functions one to one (raw
  integer pointers, sizes, a stream handle) and raise ``RhtError`` on a
  non-OK status;
* ``quantize``, ``dequantize``, ``residual_quantize``, ``residual_dequantize``,
  ``score``, ``score_sign``, ``residual_score`` and ``attention`` take torch tensors that already live on the GPU, allocate the
  outputs with ``torch.empty`` on the same device and queue the work on the
  current stream.

PyTorch is used for device memory and streams only.  There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "RhtError", "F32", "F16", "SCALE_NORM", "SCALE_SIGN_BIASED", "SCALE_SIGN_UNBIASED", "SCALE_EDEN",
    "SCALE_NORM_BETA",
    "library_path", "load", "rht_quantize", "rht_dequantize", "rht_residual_quantize",
    "rht_residual_dequantize", "rht_score", "rht_score_sign", "rht_residual_score", "rht_attention",
    "rht_attention_workspace_bytes", "rht_attention_noalloc", "rht_codebook", "rht_codebook_beta", "rht_signs",
    "rht_status_str", "rht_abi_version", "quantize", "dequantize", "residual_quantize",
    "residual_dequantize", "score", "score_sign", "residual_score", "attention", "codebook", "signs",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librht.so")

F32, F16 = 0, 1
SCALE_NORM, SCALE_SIGN_BIASED, SCALE_SIGN_UNBIASED, SCALE_EDEN, SCALE_NORM_BETA = 0, 1, 2, 3, 4
ABI_VERSION = 6

_lib = None


class RhtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, rht_status_str(status), status))


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load librht.so (built in-tree by ``build.py``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("librht.so is not built (run rotation_vector_quantization_amd/build.py "
                          "or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
    L.rht_quantize.argtypes = [vp, i32, i64, i32, i32, i32, u64, vp, vp, vp]
    L.rht_dequantize.argtypes = [vp, vp, i64, i32, i32, i32, u64, vp, i32, vp]
    L.rht_residual_quantize.argtypes = [vp, i32, i64, i32, i32, u64, vp, vp, vp, vp, vp]
    L.rht_residual_dequantize.argtypes = [vp, vp, vp, vp, i64, i32, i32, u64, vp, i32, vp]
    L.rht_score.argtypes = [vp, i32, vp, vp, i64, i32, i32, u64, vp, vp]
    L.rht_score_sign.argtypes = [vp, i32, vp, vp, i64, i32, u64, vp, vp]
    L.rht_residual_score.argtypes = [vp, i32, vp, vp, vp, vp, i64, i32, i32, u64, vp, vp]
    L.rht_attention.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i32, i32, i32, u64, u64, ctypes.c_float,
                                vp, vp, ctypes.c_size_t, vp]
    L.rht_attention_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i32, i32, i32, u64, u64,
                                        ctypes.c_float, vp, vp]
    L.rht_attention_workspace_bytes.argtypes = [i64, i32, i64, i32]
    L.rht_attention_workspace_bytes.restype = ctypes.c_size_t
    L.rht_codebook.argtypes = [i32, vp, vp]
    L.rht_codebook_beta.argtypes = [i32, i32, vp, vp]
    L.rht_signs.argtypes = [u64, i32, vp]
    L.rht_status_str.argtypes = [i32]
    L.rht_status_str.restype = ctypes.c_char_p
    L.rht_abi_version.restype = i32
    for f in ("rht_quantize", "rht_dequantize", "rht_residual_quantize", "rht_residual_dequantize",
              "rht_score", "rht_score_sign", "rht_residual_score", "rht_attention", "rht_attention_noalloc",
              "rht_codebook",
              "rht_codebook_beta", "rht_signs"):
        getattr(L, f).restype = i32
    if L.rht_abi_version() != ABI_VERSION:
        raise ImportError("librht ABI %d, binding expects %d" % (L.rht_abi_version(), ABI_VERSION))
    _lib = L
    return L


def _ok(status: int, where: str):
    if status != 0:
        raise RhtError(status, where)


# ---------------------------------------------------------------------------
# One-to-one wrappers of the C ABI (integer device pointers, stream handle).
def rht_quantize(x, xt, n, d, bits, mode, seed, codes, scale, stream=0):
    _ok(load().rht_quantize(x, xt, n, d, bits, mode, seed, codes, scale, stream), "rht_quantize")


def rht_dequantize(codes, scale, n, d, bits, mode, seed, y, yt, stream=0):
    _ok(load().rht_dequantize(codes, scale, n, d, bits, mode, seed, y, yt, stream), "rht_dequantize")


def rht_residual_quantize(x, xt, n, d, bits, seed, codes, signs, norms, res_scale, stream=0):
    _ok(load().rht_residual_quantize(x, xt, n, d, bits, seed, codes, signs, norms, res_scale, stream),
        "rht_residual_quantize")


def rht_residual_dequantize(codes, signs, norms, res_scale, n, d, bits, seed, y, yt, stream=0):
    _ok(load().rht_residual_dequantize(codes, signs, norms, res_scale, n, d, bits, seed, y, yt, stream),
        "rht_residual_dequantize")


def rht_score(q, m, codes, norms, n, d, bits, seed, logits, stream=0):
    _ok(load().rht_score(q, m, codes, norms, n, d, bits, seed, logits, stream), "rht_score")


def rht_score_sign(q, m, bits, scale, n, d, seed, logits, stream=0):
    _ok(load().rht_score_sign(q, m, bits, scale, n, d, seed, logits, stream), "rht_score_sign")


def rht_residual_score(q, m, codes, signs, norms, res_scale, n, d, bits, seed, logits, stream=0):
    _ok(load().rht_residual_score(q, m, codes, signs, norms, res_scale, n, d, bits, seed, logits, stream),
        "rht_residual_score")


def rht_attention(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits, seed_k, seed_v,
                  scale, out, workspace, workspace_bytes, stream=0):
    _ok(load().rht_attention(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits, seed_k,
                             seed_v, scale, out, workspace, workspace_bytes, stream), "rht_attention")


def rht_attention_noalloc(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits, seed_k,
                          seed_v, scale, out, stream=0):
    _ok(load().rht_attention_noalloc(q, m, k_codes, k_norms, v_codes, v_norms, heads, n, d, k_bits, v_bits,
                                     seed_k, seed_v, scale, out, stream), "rht_attention_noalloc")


def rht_attention_workspace_bytes(heads, m, n, d) -> int:
    return int(load().rht_attention_workspace_bytes(heads, m, n, d))


def rht_codebook(bits: int):
    """(levels[2^bits], thresholds[2^bits - 1]) as float32 numpy arrays."""
    K = 1 << bits
    lv = np.zeros(K, np.float32)
    th = np.zeros(max(K - 1, 1), np.float32)
    _ok(load().rht_codebook(bits, lv.ctypes.data_as(ctypes.c_void_p), th.ctypes.data_as(ctypes.c_void_p)),
        "rht_codebook")
    return lv, th[: K - 1]


def rht_codebook_beta(bits: int, d: int):
    """The exact finite-d codebook: (levels[2^bits], thresholds[2^bits - 1]) float32."""
    K = 1 << bits
    lv = np.zeros(K, np.float32)
    th = np.zeros(max(K - 1, 1), np.float32)
    _ok(load().rht_codebook_beta(bits, d, lv.ctypes.data_as(ctypes.c_void_p), th.ctypes.data_as(ctypes.c_void_p)),
        "rht_codebook_beta")
    return lv, th[: K - 1]


def rht_signs(seed: int, d: int) -> np.ndarray:
    s = np.zeros(d, np.int8)
    _ok(load().rht_signs(seed, d, s.ctypes.data_as(ctypes.c_void_p)), "rht_signs")
    return s


def rht_status_str(status: int) -> str:
    return load().rht_status_str(status).decode()


def rht_abi_version() -> int:
    return int(load().rht_abi_version())


codebook = rht_codebook
signs = rht_signs


# ---------------------------------------------------------------------------
# Torch conveniences: device tensors in, freshly allocated device tensors out.
def _torch():
    import torch
    return torch


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    raise TypeError("expected float32 or float16, got %s" % t.dtype)


def _check_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("librht works on GPU tensors only (got a %s tensor)" % t.device)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def quantize(x, bits: int, seed: int, mode: int = SCALE_NORM):
    """x [n][d] fp32/fp16 on the GPU -> (codes uint8 [n][bits*d/8], scale fp32 [n])."""
    torch = _torch()
    _check_gpu(x)
    n, d = x.shape
    codes = torch.empty((n, bits * d // 8), dtype=torch.uint8, device=x.device)
    scale = torch.empty((n,), dtype=torch.float32, device=x.device)
    rht_quantize(x.data_ptr(), _dtype_code(x), n, d, bits, mode, seed, codes.data_ptr(),
                 scale.data_ptr(), _stream(x.device))
    return codes, scale


def dequantize(codes, scale, d: int, bits: int, seed: int, mode: int = SCALE_NORM, dtype=None):
    torch = _torch()
    _check_gpu(codes, scale)
    dtype = dtype or torch.float32
    n = scale.shape[0]
    y = torch.empty((n, d), dtype=dtype, device=codes.device)
    rht_dequantize(codes.data_ptr(), scale.data_ptr(), n, d, bits, mode, seed, y.data_ptr(),
                   _dtype_code(y), _stream(codes.device))
    return y


def residual_quantize(x, bits: int, seed: int):
    """-> (codes [n][(bits-1)d/8], signs [n][d/8], norms [n], res_scale [n])."""
    torch = _torch()
    _check_gpu(x)
    n, d = x.shape
    codes = torch.empty((n, (bits - 1) * d // 8), dtype=torch.uint8, device=x.device)
    sg = torch.empty((n, d // 8), dtype=torch.uint8, device=x.device)
    norms = torch.empty((n,), dtype=torch.float32, device=x.device)
    rs = torch.empty((n,), dtype=torch.float32, device=x.device)
    rht_residual_quantize(x.data_ptr(), _dtype_code(x), n, d, bits, seed, codes.data_ptr(),
                          sg.data_ptr(), norms.data_ptr(), rs.data_ptr(), _stream(x.device))
    return codes, sg, norms, rs


def residual_dequantize(codes, sg, norms, rs, d: int, bits: int, seed: int, dtype=None):
    torch = _torch()
    _check_gpu(codes, sg, norms, rs)
    dtype = dtype or torch.float32
    n = norms.shape[0]
    y = torch.empty((n, d), dtype=dtype, device=codes.device)
    rht_residual_dequantize(codes.data_ptr(), sg.data_ptr(), norms.data_ptr(), rs.data_ptr(), n, d,
                            bits, seed, y.data_ptr(), _dtype_code(y), _stream(codes.device))
    return y


def score(q, codes, norms, d: int, bits: int, seed: int):
    """q [m][d] fp32 (m <= 64) against MSE-coded keys -> logits fp32 [m][n]."""
    torch = _torch()
    _check_gpu(q, codes, norms)
    m, n = q.shape[0], norms.shape[0]
    logits = torch.empty((m, n), dtype=torch.float32, device=q.device)
    rht_score(q.data_ptr(), m, codes.data_ptr(), norms.data_ptr(), n, d, bits, seed,
              logits.data_ptr(), _stream(q.device))
    return logits


def score_sign(q, bits, scale, d: int, seed: int):
    """q [m][d] fp32 (m <= 64) against sign-coded keys -> logits fp32 [m][n]."""
    torch = _torch()
    _check_gpu(q, bits, scale)
    m, n = q.shape[0], scale.shape[0]
    logits = torch.empty((m, n), dtype=torch.float32, device=q.device)
    rht_score_sign(q.data_ptr(), m, bits.data_ptr(), scale.data_ptr(), n, d, seed, logits.data_ptr(),
                   _stream(q.device))
    return logits


def residual_score(q, codes, signs, norms, res_scale, d: int, bits: int, seed: int):
    """q [m][d] fp32 (m <= 64) against residual-chain-coded keys -> logits fp32 [m][n]."""
    torch = _torch()
    _check_gpu(q, codes, signs, norms, res_scale)
    m, n = q.shape[0], norms.shape[0]
    logits = torch.empty((m, n), dtype=torch.float32, device=q.device)
    rht_residual_score(q.data_ptr(), m, codes.data_ptr(), signs.data_ptr(), norms.data_ptr(),
                       res_scale.data_ptr(), n, d, bits, seed, logits.data_ptr(), _stream(q.device))
    return logits


def attention(q, k_codes, k_norms, v_codes, v_norms, k_bits: int, v_bits: int, seed_k: int, seed_v: int,
              scale: float, workspace=None):
    """q [heads][m][d] fp32 over coded keys [heads][n][k_bits*d/8] and values
    [heads][n][v_bits*d/8] -> out fp32 [heads][m][d].  A workspace tensor of at
    least rht_attention_workspace_bytes bytes may be passed in."""
    torch = _torch()
    _check_gpu(q, k_codes, k_norms, v_codes, v_norms)
    heads, m, d = q.shape
    n = k_norms.shape[1]
    if (tuple(k_codes.shape) != (heads, n, k_bits * d // 8) or tuple(v_codes.shape) != (heads, n, v_bits * d // 8)
            or tuple(k_norms.shape) != (heads, n) or tuple(v_norms.shape) != (heads, n)):
        raise ValueError("attention: code and norm shapes do not match q [heads][m][d], k_bits and v_bits")
    out = torch.empty((heads, m, d), dtype=torch.float32, device=q.device)
    need = rht_attention_workspace_bytes(heads, m, n, d)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    rht_attention(q.data_ptr(), m, k_codes.data_ptr(), k_norms.data_ptr(), v_codes.data_ptr(),
                  v_norms.data_ptr(), heads, n, d, k_bits, v_bits, seed_k, seed_v, scale, out.data_ptr(),
                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q.device))
    return out
