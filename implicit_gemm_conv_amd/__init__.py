"""Python binding of libigc (include/igc.h): argument marshalling only.

Every function here forwards to the C entry point of the same name in
implicit_gemm_conv_amd/libigc.so and returns its igc_status_t as an int.
Tensor arguments may be torch tensors (their data_ptr() is passed) or plain
integer device addresses.  `stream` defaults to torch's current HIP stream.
All computation happens in the HIP kernels; there is no fallback: if the
library is not built, every call raises.

Build it with `python -m implicit_gemm_conv_amd.build` (or __graft_entry__.build()).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libigc.so")

IGC_OK, IGC_ERR_INVALID_VALUE, IGC_ERR_MISALIGNED, IGC_ERR_UNSUPPORTED, IGC_ERR_HIP = range(5)
ROW_MAJOR, COL_MAJOR = 0, 1
OUT_F32, OUT_BF16, OUT_F16 = 0, 1, 2
OUT_CODES = {"f32": OUT_F32, "bf16": OUT_BF16, "f16": OUT_F16}


class IgcError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(status_string(status))


class Tune(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int), ("bn", ctypes.c_int), ("bk", ctypes.c_int), ("pipe_depth", ctypes.c_int),
                ("waves", ctypes.c_int), ("mfma", ctypes.c_int), ("half_stage", ctypes.c_int),
                ("loader_waves", ctypes.c_int), ("k_splits", ctypes.c_int), ("stream_k", ctypes.c_int)]

    def astuple(self):
        """(bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves): the compiled configuration."""
        return (self.bm, self.bn, self.bk, self.pipe_depth, self.waves, self.mfma or 32, self.half_stage,
                self.loader_waves or self.waves)


_lib = None


def lib():
    """The loaded libigc.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m implicit_gemm_conv_amd.build`")
        # torch ships its own copy of the HIP runtime; load it first so that the
        # library binds to the same runtime that allocated the tensors passed in
        # (with two runtimes in one process, launches on torch's memory fail).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        gemm = [i64, i64, i64, p, i64, i32, p, i64, i32, p, i64, i32]
        conv = [i32] * 13 + [p, p, p, i32]
        for name, args in (("gemm_bf16", gemm + [p]), ("gemm_fp16", gemm + [p]),
                           ("gemm_bf16_ex", gemm + [ctypes.POINTER(Tune), p]),
                           ("gemm_fp16_ex", gemm + [ctypes.POINTER(Tune), p]),
                           ("conv2d_nhwc_implicit_gemm", conv + [p]),
                           ("conv2d_nhwc_implicit_gemm_fp16", conv + [p]),
                           ("conv2d_nhwc_implicit_gemm_ex", conv + [i32, ctypes.POINTER(Tune), p])):
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        L.igc_tune_supported.argtypes = [ctypes.POINTER(Tune)]
        L.igc_tune_supported.restype = i32
        L.igc_default_tune.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Tune)]
        L.igc_default_tune.restype = i32
        L.igc_tune_count.argtypes = []
        L.igc_tune_count.restype = i32
        L.igc_tune_get.argtypes = [i32, ctypes.POINTER(Tune)]
        L.igc_tune_get.restype = i32
        L.igc_tune_lds_bytes.argtypes = [ctypes.POINTER(Tune)]
        L.igc_tune_lds_bytes.restype = i64
        L.igc_status_string.argtypes = [i32]
        L.igc_status_string.restype = ctypes.c_char_p
        L.igc_ring_schedule.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_int), i32]
        L.igc_ring_schedule.restype = i32
        L.igc_probe_mfma.argtypes = [i32, i32, i32, i32, p, i64, p, i64, p]
        L.igc_probe_mfma.restype = i32
        L.igc_probe_dma.argtypes = [i32, i32, p, p, i64, p, i64, p]
        L.igc_probe_dma.restype = i32
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return ctypes.c_void_p(x.data_ptr())
    return ctypes.c_void_p(int(x))


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _tune(tune):
    if tune is None:
        return None
    if isinstance(tune, Tune):
        return ctypes.byref(tune)
    return ctypes.byref(Tune(*tune))


def gemm_bf16(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, stream=None):
    return lib().gemm_bf16(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _stream(stream))


def gemm_fp16(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, stream=None):
    return lib().gemm_fp16(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _stream(stream))


def gemm_bf16_ex(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune=None, stream=None):
    return lib().gemm_bf16_ex(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _tune(tune),
                              _stream(stream))


def gemm_fp16_ex(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune=None, stream=None):
    return lib().gemm_fp16_ex(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _tune(tune),
                              _stream(stream))


def conv2d_nhwc_implicit_gemm(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                              y_type, stream=None):
    return lib().conv2d_nhwc_implicit_gemm(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w,
                                           _ptr(x), _ptr(w), _ptr(y), y_type, _stream(stream))


def conv2d_nhwc_implicit_gemm_fp16(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                                   y_type, stream=None):
    return lib().conv2d_nhwc_implicit_gemm_fp16(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h,
                                                dil_w, _ptr(x), _ptr(w), _ptr(y), y_type, _stream(stream))


def conv2d_nhwc_implicit_gemm_ex(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                                 y_type, fp16=0, tune=None, stream=None):
    return lib().conv2d_nhwc_implicit_gemm_ex(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w,
                                              _ptr(x), _ptr(w), _ptr(y), y_type, int(fp16), _tune(tune),
                                              _stream(stream))


def igc_tune_supported(tune):
    return lib().igc_tune_supported(_tune(tune))


def igc_default_tune(M, N, K, conv=0):
    """The Tune the library picks for an M x N x K problem (conv: implicit-GEMM view)."""
    t = Tune()
    if not lib().igc_default_tune(M, N, K, int(conv), ctypes.byref(t)):
        raise ValueError("bad shape")
    return t


def igc_tune_count():
    return lib().igc_tune_count()


def igc_tune_get(i):
    t = Tune()
    return t if lib().igc_tune_get(i, ctypes.byref(t)) else None


def igc_tune_lds_bytes(tune):
    return lib().igc_tune_lds_bytes(_tune(tune))


def tunes():
    """All compiled (bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves) configurations."""
    return [igc_tune_get(i).astuple() for i in range(igc_tune_count())]


def igc_status_string(status):
    return lib().igc_status_string(int(status)).decode()


status_string = igc_status_string


def igc_ring_schedule(pipe_depth, k_tiles, half_stage=0):
    """The mainloop's event list [(kind, tile, operand, x), ...] (see include/igc.h)."""
    n = lib().igc_ring_schedule(pipe_depth, half_stage, k_tiles, None, 0)
    if n < 0:
        raise ValueError("bad ring parameters")
    buf = (ctypes.c_int * (4 * max(n, 1)))()
    lib().igc_ring_schedule(pipe_depth, half_stage, k_tiles, buf, n)
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n)]


def igc_probe_mfma(mfma, waves, iters, grid, sink, sink_bytes, clk, clk_bytes, stream=None):
    return lib().igc_probe_mfma(mfma, waves, iters, grid, _ptr(sink), sink_bytes, _ptr(clk), clk_bytes,
                                _stream(stream))


def igc_probe_dma(bk, operands, A, B, bytes_each, clk, clk_bytes, stream=None):
    return lib().igc_probe_dma(bk, operands, _ptr(A), _ptr(B), bytes_each, _ptr(clk), clk_bytes, _stream(stream))


def check(status):
    """Raises IgcError unless status is IGC_OK."""
    if status != IGC_OK:
        raise IgcError(status)
