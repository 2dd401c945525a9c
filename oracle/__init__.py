"""CPU oracle for the tiled GEMM and the NHWC implicit-GEMM convolution.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline leg may import this package.  It shares no code with the HIP library
and never imports it.

Functions evaluate the definitions directly in fp64 from the stored 16-bit
input bits (igc_oracle.c states the formulas and the passages they follow):

* gemm(...)               -> (C, S)  every output, C[i,j] = sum_k a_ik b_kj
* gemm_sample(...)        -> (c, s)  selected (row, col) outputs only
* conv2d_nhwc(...)        -> (y, S)  direct convolution, every output
* conv2d_nhwc_sample(...) -> (y, s)  selected flat NPQK outputs only
* conv2d_dgrad_nhwc(...)  -> (dx, S) data gradient (NHWC) from dy (NPQK) and w (KRSC)
* conv2d_dgrad_nhwc_sample(...)     selected flat NHWC dx outputs only
* conv2d_wgrad_nhwc(...)  -> (dw, S) filter gradient (KRSC) from x (NHWC) and dy (NPQK)
* conv2d_wgrad_nhwc_sample(...)     selected flat KRSC dw outputs only
* decode(bits, dtype)     -> exact float64 value of one bf16/fp16 pattern

S is sum |a*b| over the same terms; it scales the error bound.  After each
call, `last_threads` holds the number of CPU threads the oracle used.

Parity pins: every function here is checked against closed forms, brute force
in exact rational arithmetic, independent library routines and hand-worked
fixtures by tests/test_oracle_pins.py; tests/test_oracle_mutants.py shows those
pins catch planted mistakes.
"""
import ctypes
import os

import numpy as np

from .build import LIB, SRC, build as _build

BF16, FP16 = 0, 1
ROW_MAJOR, COL_MAJOR = 0, 1


def _bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are raw 16-bit patterns (numpy uint16)")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None and a.size else None


def conv_out_hw(H, W, R, S, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1):
    return (H + 2 * ph - dh * (R - 1) - 1) // sh + 1, (W + 2 * pw - dw * (S - 1) - 1) // sw + 1


class Oracle:
    """Binding of one compiled copy of igc_oracle.c."""

    def __init__(self, path=LIB):
        lib = ctypes.CDLL(path)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_decode.argtypes = [ctypes.c_uint16, i32]
        lib.oracle_decode.restype = ctypes.c_double
        lib.oracle_gemm.argtypes = [i64, i64, i64, p, i64, i32, p, i64, i32, i32, p, p, i32]
        lib.oracle_gemm.restype = i32
        lib.oracle_gemm_sample.argtypes = [i64, i64, i64, p, i64, i32, p, i64, i32, i32, i64, p, p, p, p, i32]
        lib.oracle_gemm_sample.restype = i32
        lib.oracle_conv2d_nhwc.argtypes = [i64] * 13 + [p, p, i32, p, p, i32]
        lib.oracle_conv2d_nhwc.restype = i32
        lib.oracle_conv2d_nhwc_sample.argtypes = [i64] * 13 + [p, p, i32, i64, p, p, p, i32]
        lib.oracle_conv2d_nhwc_sample.restype = i32
        for name in ("oracle_conv2d_dgrad_nhwc", "oracle_conv2d_wgrad_nhwc"):
            getattr(lib, name).argtypes = [i64] * 13 + [p, p, i32, p, p, i32]
            getattr(lib, name).restype = i32
        for name in ("oracle_conv2d_dgrad_nhwc_sample", "oracle_conv2d_wgrad_nhwc_sample"):
            getattr(lib, name).argtypes = [i64] * 13 + [p, p, i32, i64, p, p, p, i32]
            getattr(lib, name).restype = i32
        self.lib = lib
        self.last_threads = 0

    def _check(self, rc):
        if rc < 0:
            raise ValueError(f"oracle rejected the arguments (code {rc})")
        self.last_threads = rc
        return rc

    def decode(self, bits, dtype):
        return self.lib.oracle_decode(int(bits), int(dtype))

    def gemm(self, M, N, K, A, lda, a_layout, B, ldb, b_layout, dtype, threads=0):
        A, B = _bits(A), _bits(B)
        C = np.empty((M, N), np.float64)
        S = np.empty((M, N), np.float64)
        self._check(self.lib.oracle_gemm(M, N, K, _ptr(A), lda, a_layout, _ptr(B), ldb, b_layout, dtype,
                                         _ptr(C), _ptr(S), threads))
        return C, S

    def gemm_sample(self, M, N, K, A, lda, a_layout, B, ldb, b_layout, dtype, rows, cols, threads=0):
        A, B = _bits(A), _bits(B)
        rows = np.ascontiguousarray(rows, np.int64)
        cols = np.ascontiguousarray(cols, np.int64)
        c = np.empty(rows.shape, np.float64)
        s = np.empty(rows.shape, np.float64)
        self._check(self.lib.oracle_gemm_sample(M, N, K, _ptr(A), lda, a_layout, _ptr(B), ldb, b_layout, dtype,
                                                rows.size, _ptr(rows), _ptr(cols), _ptr(c), _ptr(s), threads))
        return c, s

    def conv2d_nhwc(self, N, H, W, C, K, R, S, x, w, dtype, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, threads=0):
        x, w = _bits(x), _bits(w)
        P, Q = conv_out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw)
        y = np.empty((N, P, Q, K), np.float64)
        ys = np.empty((N, P, Q, K), np.float64)
        self._check(self.lib.oracle_conv2d_nhwc(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, _ptr(x), _ptr(w),
                                                dtype, _ptr(y), _ptr(ys), threads))
        return y, ys

    def conv2d_nhwc_sample(self, N, H, W, C, K, R, S, x, w, dtype, idx, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1,
                           threads=0):
        x, w = _bits(x), _bits(w)
        idx = np.ascontiguousarray(idx, np.int64)
        y = np.empty(idx.shape, np.float64)
        ys = np.empty(idx.shape, np.float64)
        self._check(self.lib.oracle_conv2d_nhwc_sample(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, _ptr(x),
                                                       _ptr(w), dtype, idx.size, _ptr(idx), _ptr(y), _ptr(ys),
                                                       threads))
        return y, ys


    def conv2d_dgrad_nhwc(self, N, H, W, C, K, R, S, dy, w, dtype, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, threads=0):
        """dx[N, H, W, C] and its |.|-sum from dy[N, P, Q, K] and w[K, R, S, C] (bit arrays)."""
        dy, w = _bits(dy), _bits(w)
        dx = np.empty((N, H, W, C), np.float64)
        dxs = np.empty((N, H, W, C), np.float64)
        self._check(self.lib.oracle_conv2d_dgrad_nhwc(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, _ptr(dy), _ptr(w),
                                                      dtype, _ptr(dx), _ptr(dxs), threads))
        return dx, dxs

    def conv2d_dgrad_nhwc_sample(self, N, H, W, C, K, R, S, dy, w, dtype, idx, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1,
                                 threads=0):
        dy, w = _bits(dy), _bits(w)
        idx = np.ascontiguousarray(idx, np.int64)
        v = np.empty(idx.shape, np.float64)
        vs = np.empty(idx.shape, np.float64)
        self._check(self.lib.oracle_conv2d_dgrad_nhwc_sample(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, _ptr(dy),
                                                             _ptr(w), dtype, idx.size, _ptr(idx), _ptr(v), _ptr(vs),
                                                             threads))
        return v, vs

    def conv2d_wgrad_nhwc(self, N, H, W, C, K, R, S, x, dy, dtype, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, threads=0):
        """dw[K, R, S, C] and its |.|-sum from x[N, H, W, C] and dy[N, P, Q, K] (bit arrays)."""
        x, dy = _bits(x), _bits(dy)
        g = np.empty((K, R, S, C), np.float64)
        gs = np.empty((K, R, S, C), np.float64)
        self._check(self.lib.oracle_conv2d_wgrad_nhwc(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, _ptr(x), _ptr(dy),
                                                      dtype, _ptr(g), _ptr(gs), threads))
        return g, gs

    def conv2d_wgrad_nhwc_sample(self, N, H, W, C, K, R, S, x, dy, dtype, idx, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1,
                                 threads=0):
        x, dy = _bits(x), _bits(dy)
        idx = np.ascontiguousarray(idx, np.int64)
        v = np.empty(idx.shape, np.float64)
        vs = np.empty(idx.shape, np.float64)
        self._check(self.lib.oracle_conv2d_wgrad_nhwc_sample(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, _ptr(x),
                                                             _ptr(dy), dtype, idx.size, _ptr(idx), _ptr(v), _ptr(vs),
                                                             threads))
        return v, vs


_default = None


def default():
    """The oracle built from oracle/igc_oracle.c (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            _build()
        _default = Oracle(LIB)
    return _default


def decode(bits, dtype):
    return default().decode(bits, dtype)


def gemm(*a, **k):
    return default().gemm(*a, **k)


def gemm_sample(*a, **k):
    return default().gemm_sample(*a, **k)


def conv2d_nhwc(*a, **k):
    return default().conv2d_nhwc(*a, **k)


def conv2d_nhwc_sample(*a, **k):
    return default().conv2d_nhwc_sample(*a, **k)


def last_threads():
    return default().last_threads


def conv2d_dgrad_nhwc(*a, **k):
    return default().conv2d_dgrad_nhwc(*a, **k)


def conv2d_dgrad_nhwc_sample(*a, **k):
    return default().conv2d_dgrad_nhwc_sample(*a, **k)


def conv2d_wgrad_nhwc(*a, **k):
    return default().conv2d_wgrad_nhwc(*a, **k)


def conv2d_wgrad_nhwc_sample(*a, **k):
    return default().conv2d_wgrad_nhwc_sample(*a, **k)
