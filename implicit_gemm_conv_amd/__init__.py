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
OP_GEMM, OP_CONV_FPROP, OP_CONV_DGRAD, OP_CONV_WGRAD = range(4)

# Every exported entry point (include/igc.h), for the load check.
EXPORTS = (
    "gemm_bf16", "gemm_fp16", "gemm_bf16_ex", "gemm_fp16_ex", "gemm_bf16_noalloc",
    "conv2d_nhwc_implicit_gemm", "conv2d_nhwc_implicit_gemm_fp16", "conv2d_nhwc_implicit_gemm_ex",
    "conv2d_nhwc_implicit_gemm_fp16_ex",
    "conv2d_nhwc_dgrad_implicit_gemm", "conv2d_nhwc_dgrad_implicit_gemm_fp16", "conv2d_nhwc_dgrad_implicit_gemm_ex",
    "conv2d_nhwc_dgrad_implicit_gemm_fp16_ex",
    "conv2d_nhwc_wgrad_implicit_gemm", "conv2d_nhwc_wgrad_implicit_gemm_fp16", "conv2d_nhwc_wgrad_implicit_gemm_ex",
    "conv2d_nhwc_wgrad_implicit_gemm_fp16_ex",
    "igc_workspace_bytes", "igc_tune_supported", "igc_default_tune", "igc_tune_count", "igc_tune_get",
    "igc_tune_scope", "igc_tune_lds_bytes", "igc_status_string", "igc_take_device_error", "igc_debug_stream_k",
    "igc_pool_allocations", "igc_ring_schedule", "igc_lds_chunk", "igc_stage_slot",
)


class IgcError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(status_string(status))


class Tune(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int), ("bn", ctypes.c_int), ("bk", ctypes.c_int), ("pipe_depth", ctypes.c_int),
                ("waves", ctypes.c_int), ("mfma", ctypes.c_int), ("half_stage", ctypes.c_int),
                ("loader_waves", ctypes.c_int), ("k_splits", ctypes.c_int), ("stream_k", ctypes.c_int),
                ("ring_sync", ctypes.c_int), ("sk_hybrid", ctypes.c_int)]

    def astuple(self):
        """(bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves, ring_sync): the compiled configuration."""
        return (self.bm, self.bn, self.bk, self.pipe_depth, self.waves, self.mfma or 32, self.half_stage,
                self.loader_waves or self.waves, self.ring_sync)


def tune(cfg, k_splits=0, stream_k=0, sk_hybrid=0):
    """A Tune from a compiled configuration tuple (bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves
    [, ring_sync]) and a schedule."""
    cfg = tuple(cfg)
    ring_sync = cfg[8] if len(cfg) > 8 else 0
    return Tune(*cfg[:8], k_splits, stream_k, ring_sync, sk_hybrid)


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
        tp = ctypes.POINTER(Tune)
        gemm = [i64, i64, i64, p, i64, i32, p, i64, i32, p, i64, i32]
        conv = [i32] * 13 + [p, p, p, i32]
        protos = {"gemm_bf16": gemm + [p], "gemm_fp16": gemm + [p], "gemm_bf16_noalloc": gemm + [p],
                  "gemm_bf16_ex": gemm + [tp, p, i64, p], "gemm_fp16_ex": gemm + [tp, p, i64, p]}
        for base in ("conv2d_nhwc_implicit_gemm", "conv2d_nhwc_dgrad_implicit_gemm", "conv2d_nhwc_wgrad_implicit_gemm"):
            protos[base] = conv + [p]
            protos[base + "_fp16"] = conv + [p]
            protos[base + "_ex"] = conv + [tp, p, i64, p]
            protos[base + "_fp16_ex"] = conv + [tp, p, i64, p]
        for name, args in protos.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        L.igc_workspace_bytes.argtypes = [i32, i64, i64, i64, tp]
        L.igc_workspace_bytes.restype = i64
        L.igc_tune_supported.argtypes = [tp]
        L.igc_tune_supported.restype = i32
        L.igc_default_tune.argtypes = [i32, i64, i64, i64, tp]
        L.igc_default_tune.restype = i32
        L.igc_tune_count.argtypes = []
        L.igc_tune_count.restype = i32
        L.igc_tune_get.argtypes = [i32, tp]
        L.igc_tune_get.restype = i32
        L.igc_tune_scope.argtypes = [i32]
        L.igc_tune_scope.restype = i32
        L.igc_tune_lds_bytes.argtypes = [tp]
        L.igc_tune_lds_bytes.restype = i64
        L.igc_status_string.argtypes = [i32]
        L.igc_status_string.restype = ctypes.c_char_p
        L.igc_take_device_error.argtypes = [ctypes.POINTER(ctypes.c_int)]
        L.igc_take_device_error.restype = i32
        L.igc_debug_stream_k.argtypes = [i32, i32]
        L.igc_debug_stream_k.restype = None
        L.igc_pool_allocations.argtypes = []
        L.igc_pool_allocations.restype = i64
        L.igc_ring_schedule.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_int), i32]
        L.igc_ring_schedule.restype = i32
        L.igc_lds_chunk.argtypes = [i32, i32, i32, i32]
        L.igc_lds_chunk.restype = i32
        L.igc_stage_slot.argtypes = [i32, i32, i32]
        L.igc_stage_slot.restype = i32
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return ctypes.c_void_p(x.data_ptr())
    return ctypes.c_void_p(int(x))


def _nbytes(x):
    if x is None:
        return 0
    if hasattr(x, "numel"):
        return x.numel() * x.element_size()
    raise TypeError("pass workspace_bytes with a raw workspace address")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _tune(t):
    if t is None:
        return None
    if isinstance(t, Tune):
        return ctypes.byref(t)
    t = tuple(t)
    return ctypes.byref(Tune(*t) if len(t) >= 10 else tune(t))


def gemm_bf16(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, stream=None):
    return lib().gemm_bf16(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _stream(stream))


def gemm_fp16(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, stream=None):
    return lib().gemm_fp16(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _stream(stream))


def gemm_bf16_noalloc(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, stream=None):
    return lib().gemm_bf16_noalloc(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type,
                                   _stream(stream))


def gemm_bf16_ex(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune=None, workspace=None, workspace_bytes=None,
                 stream=None):
    wsb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    return lib().gemm_bf16_ex(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _tune(tune),
                              _ptr(workspace), wsb, _stream(stream))


def gemm_fp16_ex(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune=None, workspace=None, workspace_bytes=None,
                 stream=None):
    wsb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    return lib().gemm_fp16_ex(M, N, K, _ptr(A), lda, la, _ptr(B), ldb, lb, _ptr(C), ldc, c_type, _tune(tune),
                              _ptr(workspace), wsb, _stream(stream))


def _conv_plain(name):
    def call(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, in0, in1, out, out_type,
             stream=None):
        return getattr(lib(), name)(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, _ptr(in0),
                                    _ptr(in1), _ptr(out), out_type, _stream(stream))
    call.__name__ = name
    return call


def _conv_ex(name):
    def call(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, in0, in1, out, out_type,
             tune=None, workspace=None, workspace_bytes=None, stream=None):
        wsb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
        return getattr(lib(), name)(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, _ptr(in0),
                                    _ptr(in1), _ptr(out), out_type, _tune(tune), _ptr(workspace), wsb,
                                    _stream(stream))
    call.__name__ = name
    return call


# forward: (x, w) -> y;  data gradient: (dy, w) -> dx;  filter gradient: (x, dy) -> dw
conv2d_nhwc_implicit_gemm = _conv_plain("conv2d_nhwc_implicit_gemm")
conv2d_nhwc_implicit_gemm_fp16 = _conv_plain("conv2d_nhwc_implicit_gemm_fp16")
conv2d_nhwc_implicit_gemm_ex = _conv_ex("conv2d_nhwc_implicit_gemm_ex")
conv2d_nhwc_implicit_gemm_fp16_ex = _conv_ex("conv2d_nhwc_implicit_gemm_fp16_ex")
conv2d_nhwc_dgrad_implicit_gemm = _conv_plain("conv2d_nhwc_dgrad_implicit_gemm")
conv2d_nhwc_dgrad_implicit_gemm_fp16 = _conv_plain("conv2d_nhwc_dgrad_implicit_gemm_fp16")
conv2d_nhwc_dgrad_implicit_gemm_ex = _conv_ex("conv2d_nhwc_dgrad_implicit_gemm_ex")
conv2d_nhwc_dgrad_implicit_gemm_fp16_ex = _conv_ex("conv2d_nhwc_dgrad_implicit_gemm_fp16_ex")
conv2d_nhwc_wgrad_implicit_gemm = _conv_plain("conv2d_nhwc_wgrad_implicit_gemm")
conv2d_nhwc_wgrad_implicit_gemm_fp16 = _conv_plain("conv2d_nhwc_wgrad_implicit_gemm_fp16")
conv2d_nhwc_wgrad_implicit_gemm_ex = _conv_ex("conv2d_nhwc_wgrad_implicit_gemm_ex")
conv2d_nhwc_wgrad_implicit_gemm_fp16_ex = _conv_ex("conv2d_nhwc_wgrad_implicit_gemm_fp16_ex")


def conv_out_hw(H, W, R, S, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1):
    """Output size (P, Q) of the forward convolution."""
    return (H + 2 * ph - dh * (R - 1) - 1) // sh + 1, (W + 2 * pw - dw * (S - 1) - 1) // sw + 1


def conv_gemm_view(op, N, H, W, C, K, R, S, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1):
    """(M, N_gemm, K_gemm) of a convolution operation, as include/igc.h defines them."""
    P, Q = conv_out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw)
    if op == OP_CONV_FPROP:
        return N * P * Q, K, R * S * C
    if op == OP_CONV_DGRAD:
        return N * H * W, C, R * S * K
    return K, R * S * C, N * P * Q


def igc_workspace_bytes(op, M, N, K, tune=None):
    return lib().igc_workspace_bytes(op, M, N, K, _tune(tune))


def igc_tune_supported(t):
    return lib().igc_tune_supported(_tune(t))


def igc_default_tune(M, N, K, op=OP_GEMM):
    """The Tune the library picks for operation `op` with GEMM view M x N x K."""
    t = Tune()
    if not lib().igc_default_tune(op, M, N, K, ctypes.byref(t)):
        raise ValueError("bad shape")
    return t


def igc_tune_count():
    return lib().igc_tune_count()


def igc_tune_get(i):
    t = Tune()
    return t if lib().igc_tune_get(i, ctypes.byref(t)) else None


SCOPE_ALL, SCOPE_STREAM_K, SCOPE_CONV_FPROP = 1, 2, 4


def igc_tune_scope(i):
    return lib().igc_tune_scope(i)


def igc_tune_lds_bytes(t):
    return lib().igc_tune_lds_bytes(_tune(t))


def tunes(scope=0):
    """Compiled (bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves, ring_sync) configurations whose
    scope includes every bit of `scope` (SCOPE_ALL: every type, layout and operation; SCOPE_STREAM_K;
    SCOPE_CONV_FPROP: the complete forward convolution)."""
    return [igc_tune_get(i).astuple() for i in range(igc_tune_count()) if igc_tune_scope(i) & scope == scope]


def igc_status_string(status):
    return lib().igc_status_string(int(status)).decode()


status_string = igc_status_string


def igc_take_device_error():
    """The current device's error word (then cleared); synchronises the device."""
    v = ctypes.c_int(0)
    check(lib().igc_take_device_error(ctypes.byref(v)))
    return v.value


def igc_debug_stream_k(spin_limit=0, drop_workgroup=-1):
    lib().igc_debug_stream_k(spin_limit, drop_workgroup)


def igc_pool_allocations():
    return lib().igc_pool_allocations()


def igc_ring_schedule(pipe_depth, k_tiles, half_stage=0):
    """The mainloop's event list [(kind, tile, operand, x), ...] (see include/igc.h)."""
    n = lib().igc_ring_schedule(pipe_depth, half_stage, k_tiles, None, 0)
    if n < 0:
        raise ValueError("bad ring parameters")
    buf = (ctypes.c_int * (4 * max(n, 1)))()
    lib().igc_ring_schedule(pipe_depth, half_stage, k_tiles, buf, n)
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n)]


def igc_lds_chunk(k_contiguous, chunks_per_row, row, logical_chunk):
    return lib().igc_lds_chunk(k_contiguous, chunks_per_row, row, logical_chunk)


def igc_stage_slot(row, slot, slots_per_row):
    return lib().igc_stage_slot(row, slot, slots_per_row)


def check(status):
    """Raises IgcError unless status is IGC_OK."""
    if status != IGC_OK:
        raise IgcError(status)
