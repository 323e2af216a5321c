"""Seeded synthetic inputs for the tests, the benchmark and the smoke check.

Shared by both sides of every parity check: the same bytes feed the CPU oracle
and the HIP library. This module draws input vectors only; it contains none of
the quantizer's arithmetic. The random streams are defined in ``gen.c``.

Workloads (row-major, one vector per row; ``seed`` draws the data, ``rot_seed``
is the rotation seed the workload is quantized with):

* ``c1``  4096 x 128 fp32, N(0,1) with channels {3, 77} scaled x20; 2-bit.
* ``c2k``/``c2v``  KV-cache block, K and V each 32 layers x 8 heads x 32768
  tokens x 128 fp16 (n = 8,388,608 each): N(0,1), one seeded outlier channel
  (1% of 128, at least one) x20, every vector scaled by exp(0.5 g), g ~ N(0,1);
  4-bit.
* ``c3``  65536 x 1024 fp32 Student-t (nu = 3): z / sqrt((z1^2+z2^2+z3^2)/3);
  1-bit sign code.
* ``c4``  16 heads x 65536 tokens x 256 fp16 (n = 1,048,576): N(0,1) with 5
  seeded outlier channels (2% of 256) x30; residual chain, 3 bits in total.
* ``c5k`` 131072 x 128 fp32 keys N(0,1) (4-bit codes); ``c5q`` 64 x 128 fp32
  queries N(0,1).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libtdg.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=gnu99", "-Wall", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.tdg_subkey.argtypes = [u64, u64]
        L.tdg_subkey.restype = u64
        L.tdg_unif.argtypes = [u64, u64]
        L.tdg_unif.restype = ctypes.c_double
        L.tdg_normal.argtypes = [u64, u64]
        L.tdg_normal.restype = ctypes.c_double
        L.tdg_f32_to_f16.argtypes = [ctypes.c_float]
        L.tdg_f32_to_f16.restype = ctypes.c_uint16
        L.tdg_pick_channels.argtypes = [u64, i32, i32, vp]
        L.tdg_generate.argtypes = [i32, u64, i64, i64, i32, vp, i32, ctypes.c_double,
                                   ctypes.c_double, i32, vp, i32]
        L.tdg_generate.restype = i32
        _lib = L
    return _lib


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    d: int
    dtype: str              # "f32" or "f16"
    seed: int               # data seed
    rot_seed: int           # rotation seed used to quantize it
    bits: int
    kind: int = 0           # 0 Gaussian (+ outlier channels), 1 Student-t nu=3
    channels: tuple = ()    # explicit outlier channels
    n_outlier: int = 0      # else: this many seeded channels
    mult: float = 1.0
    lognorm_sigma: float = 0.0

    @property
    def np_dtype(self):
        return np.float16 if self.dtype == "f16" else np.float32

    def outlier_channels(self) -> np.ndarray:
        if self.channels:
            return np.array(self.channels, dtype=np.int32)
        out = np.zeros(self.n_outlier, dtype=np.int32)
        if self.n_outlier:
            lib().tdg_pick_channels(self.seed, self.d, self.n_outlier,
                                    out.ctypes.data_as(ctypes.c_void_p))
        return out


def _n_outlier(frac: float, d: int) -> int:
    return max(1, int(round(frac * d)))


WORKLOADS = {
    "c1": Workload("c1", 4096, 128, "f32", 1001, 42, 2, channels=(3, 77), mult=20.0),
    "c2k": Workload("c2k", 32 * 8 * 32768, 128, "f16", 1002, 42, 4,
                    n_outlier=_n_outlier(0.01, 128), mult=20.0, lognorm_sigma=0.5),
    "c2v": Workload("c2v", 32 * 8 * 32768, 128, "f16", 1003, 43, 4,
                    n_outlier=_n_outlier(0.01, 128), mult=20.0, lognorm_sigma=0.5),
    "c3": Workload("c3", 65536, 1024, "f32", 1004, 44, 1, kind=1),
    "c4": Workload("c4", 16 * 65536, 256, "f16", 1005, 45, 3,
                   n_outlier=_n_outlier(0.02, 256), mult=30.0),
    "c5k": Workload("c5k", 131072, 128, "f32", 1006, 46, 4),
    "c5q": Workload("c5q", 64, 128, "f32", 1007, 46, 4),
}


def generate(w: Workload, row0: int = 0, nrows: int | None = None, nthreads: int | None = None,
             out: np.ndarray | None = None) -> np.ndarray:
    """Rows [row0, row0 + nrows) of workload ``w`` as a numpy array [nrows][d]."""
    if nrows is None:
        nrows = w.n - row0
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    if out is None:
        out = np.empty((nrows, w.d), dtype=w.np_dtype)
    assert out.shape == (nrows, w.d) and out.dtype == w.np_dtype and out.flags.c_contiguous
    ch = w.outlier_channels()
    lib().tdg_generate(w.kind, w.seed, row0, nrows, w.d, ch.ctypes.data_as(ctypes.c_void_p),
                       len(ch), float(w.mult), float(w.lognorm_sigma),
                       1 if w.dtype == "f16" else 0, out.ctypes.data_as(ctypes.c_void_p), nthreads)
    return out


def generate_rows(w: Workload, rows: np.ndarray) -> np.ndarray:
    """Arbitrary (e.g. sampled) rows of ``w``, in the order given."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), w.d), dtype=w.np_dtype)
    for i, r in enumerate(rows):
        generate(w, int(r), 1, nthreads=1, out=out[i:i + 1])
    return out


def scaled(w: Workload, n: int) -> Workload:
    """The same recipe with fewer (or more) rows; rows are identical prefixes."""
    return dataclasses.replace(w, n=n)
