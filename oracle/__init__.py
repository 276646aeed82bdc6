"""CPU oracle for the additive-quantized matrix-vector product -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never does, and this package never imports
the product library: the two share no code.

The arithmetic lives in ``aqlm_oracle.c`` (plain C99, fp32 decode fold, double
matvec); this file only loads it and marshals numpy arrays.  See the C file's
header for the definitions and the readings taken where the pages are silent.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(bitrate worked examples, brute-force decode, additivity, linearity,
permutation invariance, unit vectors, hand-computed integer cases, and a
planted-mistake check that the pins fail on a broken copy).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "aqlm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
GROUP = 8

CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(out_path: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *extra_flags, _SRC, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


_lib = None


def _declare(lib):
    i64, f32p, f64p, vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_float), \
        ctypes.POINTER(ctypes.c_double), ctypes.c_void_p
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.oracle_bits_per_weight.restype = ctypes.c_double
    lib.oracle_bits_per_weight.argtypes = [ctypes.c_int] * 3
    lib.oracle_codes_bytes.restype = i64
    lib.oracle_codes_bytes.argtypes = [i64, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_half_to_float.restype = ctypes.c_float
    lib.oracle_half_to_float.argtypes = [ctypes.c_uint16]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [vp, u16p, f32p, i64, i64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int]
    lib.oracle_matvec.restype = ctypes.c_int
    lib.oracle_matvec.argtypes = [f32p, u16p, f64p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemv_rows.restype = ctypes.c_int
    lib.oracle_gemv_rows.argtypes = [vp, u16p, u16p, ctypes.POINTER(i64), i64, f64p, i64, i64,
                                     ctypes.c_int, ctypes.c_int, i64, f32p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library.  ``path`` selects another build."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as_u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("fp16 data must be float16 or uint16 bit patterns")
    return a


def _check_codes(codes, B):
    codes = np.ascontiguousarray(codes)
    want = np.uint8 if B == 8 else np.uint16
    if codes.dtype != want:
        if B == 16 and codes.dtype == np.int16:
            return codes.view(np.uint16)
        raise TypeError(f"codes for B={B} must be {want}")
    return codes


class Oracle:
    """Thin numpy front end over one build of the C oracle."""

    def __init__(self, lib=None, nthreads: int = 0):
        self.lib = lib if lib is not None else load()
        self.nthreads = nthreads

    def bits_per_weight(self, K, B, group=GROUP) -> float:
        return self.lib.oracle_bits_per_weight(K, B, group)

    def codes_bytes(self, out_features, in_features, K, B) -> int:
        return self.lib.oracle_codes_bytes(out_features, in_features, K, B)

    def half_to_float(self, h) -> np.ndarray:
        h = _as_u16(np.asarray(h)).ravel()
        f = self.lib.oracle_half_to_float
        return np.array([f(int(v)) for v in h], dtype=np.float32)

    def float_to_half(self, x) -> np.ndarray:
        x = np.asarray(x, dtype=np.float32).ravel()
        f = self.lib.oracle_float_to_half
        return np.array([f(float(v)) for v in x], dtype=np.uint16)

    def decode(self, codes, codebooks, K: int, B: int) -> np.ndarray:
        """Dense fp32 W [out][in] from codes [out][in/8][K] and codebooks [K][2^B][8]."""
        codes = _check_codes(codes, B)
        cb = _as_u16(codebooks)
        out_f, G, k2 = codes.shape
        if k2 != K or cb.shape != (K, 1 << B, GROUP):
            raise ValueError("shape mismatch")
        W = np.empty((out_f, G * GROUP), dtype=np.float32)
        rc = self.lib.oracle_decode(codes.ctypes.data, _ptr(cb, ctypes.c_uint16),
                                    _ptr(W, ctypes.c_float), out_f, G * GROUP, K, B,
                                    self.nthreads)
        if rc:
            raise ValueError("oracle_decode rejected its arguments")
        return W

    def matvec(self, W, x) -> np.ndarray:
        """Y [batch][out] in double from fp32 W [out][in] and fp16 x [batch][in]."""
        W = np.ascontiguousarray(W, dtype=np.float32)
        x = _as_u16(np.atleast_2d(x))
        out_f, in_f = W.shape
        if x.shape[1] != in_f:
            raise ValueError("shape mismatch")
        Y = np.empty((x.shape[0], out_f), dtype=np.float64)
        rc = self.lib.oracle_matvec(_ptr(W, ctypes.c_float), _ptr(x, ctypes.c_uint16),
                                    _ptr(Y, ctypes.c_double), out_f, in_f, x.shape[0],
                                    self.nthreads)
        if rc:
            raise ValueError("oracle_matvec rejected its arguments")
        return Y

    def gemv(self, codes, codebooks, x, K: int, B: int) -> np.ndarray:
        """Decode then matvec: the whole reference result Y [batch][out] in double."""
        return self.matvec(self.decode(codes, codebooks, K, B), x)

    def gemv_rows(self, codes, codebooks, x, K: int, B: int, rows) -> np.ndarray:
        """Y[:, rows] in double, decoding only the listed rows."""
        codes = _check_codes(codes, B)
        cb = _as_u16(codebooks)
        x = _as_u16(np.atleast_2d(x))
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out_f, G, _ = codes.shape
        in_f = G * GROUP
        nt = self.nthreads if self.nthreads > 0 else self.lib.oracle_max_threads()
        scratch = np.empty((max(nt, 1), in_f), dtype=np.float32)
        Y = np.empty((x.shape[0], rows.size), dtype=np.float64)
        rc = self.lib.oracle_gemv_rows(codes.ctypes.data, _ptr(cb, ctypes.c_uint16),
                                       _ptr(x, ctypes.c_uint16), _ptr(rows, ctypes.c_int64),
                                       rows.size, _ptr(Y, ctypes.c_double), out_f, in_f, K, B,
                                       x.shape[0], _ptr(scratch, ctypes.c_float), nt)
        if rc:
            raise ValueError("oracle_gemv_rows rejected its arguments")
        return Y

    def max_threads(self) -> int:
        return self.lib.oracle_max_threads()
