// igc_lib.hip -- C ABI of libigc: argument checks, instance selection, launch.
//
// Every entry point validates its arguments completely before it enqueues
// anything, then launches its kernels on the caller's stream and returns.  The
// only memory it allocates is the fp32 workspace of a K split or a stream-K
// schedule, stream-ordered from a pool the library keeps per device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "igc.h"
#include "instances.hpp"
#include "mainloop.hpp"
#include "ring.hpp"
#include "split_reduce.hpp"

// Tiles of M that one XCD walks together (its share of the tile grid is
// GROUP_M tiles tall): larger groups trade A-row reuse for B-column reuse in
// that XCD's L2.
#ifndef IGC_GROUP_M
#define IGC_GROUP_M 8
#endif

namespace igc {

static bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Workspaces come from a stream-ordered memory pool of the library's own, one
// per device, which keeps up to kPoolKeepBytes of freed memory mapped for the
// next call.  (A pool that returns its memory at every synchronisation, the
// default pool's behaviour, remaps the workspace on each call: 8-20 us per call
// for workspaces of 16-64 MB.)  The default pool is left untouched.
constexpr uint64_t kPoolKeepBytes = 256ull << 20;
constexpr int kMaxDevices = 64;

static hipMemPool_t workspace_pool() {
    static std::mutex mu;
    static hipMemPool_t pools[kMaxDevices];
    static bool tried[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!tried[dev]) {
        tried[dev] = true;
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
            uint64_t keep = kPoolKeepBytes;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
            pools[dev] = pool;
        }
        (void)hipGetLastError();  // a pool this runtime cannot create falls back below
    }
    return pools[dev];
}

// Stream-ordered workspace of `bytes` on the current device; nullptr on failure.
static void* workspace_alloc(size_t bytes, hipStream_t stream) {
    void* ptr = nullptr;
    hipMemPool_t pool = workspace_pool();
    hipError_t e = pool ? hipMallocFromPoolAsync(&ptr, bytes, pool, stream) : hipMallocAsync(&ptr, bytes, stream);
    return e == hipSuccess ? ptr : nullptr;
}

// Stream-K flags are raised to a per-call epoch, written with its complement,
// so a workspace holding flags of earlier calls (or any other data) needs no
// clearing: only the pair (epoch, ~epoch) of this call counts as raised.  The
// epoch is a call counter passed through a bijective 32-bit mix (so
// consecutive calls differ in many bits), keeping 31 bits.
static std::atomic<uint32_t> g_stream_k_calls{0};
static int next_stream_k_epoch() {
    uint32_t x = g_stream_k_calls.fetch_add(1, std::memory_order_relaxed) + 0x9e3779b9u;
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return (int)(x & 0x7fffffffu);
}

static int out_size(igc_out_t t) { return t == IGC_OUT_F32 ? 4 : 2; }

struct Plan {
    const Instance* inst = nullptr;
    int splits = 1;
    int stream_k = 0;  // persistent workgroups of a stream-K schedule (0: none)
    bool valid = true;
};

// The tile configuration and K split for one call: an explicit tune is taken as
// is (k_splits <= 1: no split); otherwise the built-in choice for the shape.
static Plan pick(const igc_tune_t* tune, bool fp16, bool a_kc, bool b_kc, bool conv, int64_t M, int64_t N,
                 int64_t K) {
    const igc_tune_t t = tune ? *tune : default_tune(M, N, K, conv);
    Plan pl;
    pl.inst = find_instance(t, fp16, a_kc, b_kc, conv);
    pl.splits = t.k_splits > 1 ? t.k_splits : 1;
    pl.stream_k = t.stream_k > 0 ? t.stream_k : 0;
    pl.valid = t.stream_k >= 0 && !(pl.splits > 1 && pl.stream_k > 0);
    return pl;
}

// Launches the mainloop (and, for a K split, the fixed-order reduction).  With
// S > 1 splits the fp32 partial tiles live in a stream-ordered workspace taken
// from the library's pool and released with hipFreeAsync after the reduction is
// enqueued, so concurrent calls on different streams never share it.
static igc_status_t launch(const Plan& pl, Params p, hipStream_t stream) {
    const Instance* inst = pl.inst;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles <= 0) return IGC_OK;
    if (pl.stream_k > 0 && p.K > 0) {
        // stream-K: K of every tile in units of one ring period; G runs of equal length
        const int64_t unit = (int64_t)inst->bk * Ring::period(Ring::units(inst->d, inst->half));
        const int64_t UT = (p.K + unit - 1) / unit;
        const int64_t G = pl.stream_k < tiles * UT ? pl.stream_k : tiles * UT;
        const size_t part_bytes = (size_t)G * inst->bm * inst->bn * sizeof(float);
        (void)hipGetLastError();
        char* ws = (char*)workspace_alloc(part_bytes + (size_t)G * 2 * sizeof(int), stream);
        if (!ws) return IGC_ERR_HIP;
        p.sk_grid = (int)G;
        p.sk_units = UT;
        p.sk_ws = (float*)ws;
        p.sk_flags = (int*)(ws + part_bytes);
        p.sk_epoch = next_stream_k_epoch();
        p.k_splits = 1;
        Params arg = p;
        void* args[] = {&arg};
        hipError_t e = hipLaunchKernel(inst->fn, dim3((unsigned)G), dim3(64 * inst->waves), args, 0, stream);
        (void)hipFreeAsync(ws, stream);
        if (e != hipSuccess) return IGC_ERR_HIP;
        return hipGetLastError() == hipSuccess ? IGC_OK : IGC_ERR_HIP;
    }
    int S = 1;
    p.k_per_split = p.K > 0 ? p.K : 1;
    if (pl.splits > 1 && p.K > 0) {
        // each split a whole number of ring periods (no padding tiles inside a split)
        const int64_t unit = (int64_t)inst->bk * Ring::period(Ring::units(inst->d, inst->half));
        const int64_t per = ((p.K + pl.splits - 1) / pl.splits + unit - 1) / unit * unit;
        S = (int)((p.K + per - 1) / per);
        p.k_per_split = per;
    }
    if (tiles * S > 0x7fffffff) return IGC_ERR_UNSUPPORTED;
    p.k_splits = S;
    (void)hipGetLastError();  // launch errors below are ours alone
    float* ws = nullptr;
    if (S > 1) {
        p.ldws = (p.N + 3) / 4 * 4;
        p.ws_stride = p.M * p.ldws;
        ws = (float*)workspace_alloc((size_t)(S * p.ws_stride) * sizeof(float), stream);
        if (!ws) return IGC_ERR_HIP;
        p.ws = ws;
    }
    Params arg = p;
    void* args[] = {&arg};
    hipError_t e = hipLaunchKernel(inst->fn, dim3((unsigned)(tiles * S)), dim3(64 * inst->waves), args, 0, stream);
    if (e == hipSuccess && S > 1)
        e = launch_split_reduce(ws, S, p.ws_stride, p.M, p.N, p.ldws, p.C, p.ldc, p.out_kind, stream);
    if (ws) (void)hipFreeAsync(ws, stream);
    if (e != hipSuccess) return IGC_ERR_HIP;
    return hipGetLastError() == hipSuccess ? IGC_OK : IGC_ERR_HIP;
}

static igc_status_t gemm_any(bool fp16, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             igc_layout_t la, const void* B, int64_t ldb, igc_layout_t lb, void* C, int64_t ldc,
                             igc_out_t ct, const igc_tune_t* tune, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0) return IGC_ERR_INVALID_VALUE;
    if ((la != IGC_ROW_MAJOR && la != IGC_COL_MAJOR) || (lb != IGC_ROW_MAJOR && lb != IGC_COL_MAJOR))
        return IGC_ERR_INVALID_VALUE;
    if (ct != IGC_OUT_F32 && ct != IGC_OUT_BF16 && ct != IGC_OUT_F16) return IGC_ERR_INVALID_VALUE;
    const bool a_kc = la == IGC_ROW_MAJOR, b_kc = lb == IGC_COL_MAJOR;
    const Plan pl = pick(tune, fp16, a_kc, b_kc, false, M, N, K);
    if (!pl.valid) return IGC_ERR_INVALID_VALUE;
    const Instance* inst = pl.inst;
    if (!inst) return IGC_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return IGC_OK;
    if (!C || ldc < N) return IGC_ERR_INVALID_VALUE;
    if (K > 0) {
        if (!A || !B) return IGC_ERR_INVALID_VALUE;
        if (lda < (a_kc ? K : M) || ldb < (b_kc ? K : N)) return IGC_ERR_INVALID_VALUE;
        if (!aligned16(A) || !aligned16(B) || (lda * 2) % 16 != 0 || (ldb * 2) % 16 != 0)
            return IGC_ERR_MISALIGNED;
        // Per-tile buffer offsets are 32-bit: one tile's rows must span < 2^31 bytes.
        if (a_kc && (inst->bm * lda + inst->bk) * 2 >= 0x7fffffffLL) return IGC_ERR_UNSUPPORTED;
        if (b_kc && (inst->bn * ldb + inst->bk) * 2 >= 0x7fffffffLL) return IGC_ERR_UNSUPPORTED;
        if (!a_kc && (inst->bk * lda + inst->bm) * 2 >= 0x7fffffffLL) return IGC_ERR_UNSUPPORTED;
        if (!b_kc && (inst->bk * ldb + inst->bn) * 2 >= 0x7fffffffLL) return IGC_ERR_UNSUPPORTED;
    }
    if (!aligned16(C) || (ldc * out_size(ct)) % 16 != 0) return IGC_ERR_MISALIGNED;

    Params p = {};
    p.A = A;
    p.B = B;
    p.C = C;
    p.M = M;
    p.N = N;
    p.K = K;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.tiles_m = (int)((M + inst->bm - 1) / inst->bm);
    p.tiles_n = (int)((N + inst->bn - 1) / inst->bn);
    if ((M + inst->bm - 1) / inst->bm > 0x7fffffff || (N + inst->bn - 1) / inst->bn > 0x7fffffff)
        return IGC_ERR_UNSUPPORTED;
    p.out_kind = (int)ct;
    p.group_m = IGC_GROUP_M;
    p.k_ragged8 = (K % 8) != 0;
    p.vec_ok = 1;
    return launch(pl, p, stream);
}

static igc_status_t conv_any(bool fp16, int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph,
                             int pw, int dh, int dw, const void* x, const void* w, void* y, igc_out_t yt,
                             const igc_tune_t* tune, hipStream_t stream) {
    if (N < 0 || K < 0 || H < 1 || W < 1 || C < 1 || R < 1 || S < 1 || sh < 1 || sw < 1 || ph < 0 || pw < 0 ||
        dh < 1 || dw < 1)
        return IGC_ERR_INVALID_VALUE;
    if (yt != IGC_OUT_F32 && yt != IGC_OUT_BF16 && yt != IGC_OUT_F16) return IGC_ERR_INVALID_VALUE;
    const int64_t hspan = (int64_t)H + 2LL * ph - (int64_t)dh * (R - 1) - 1;
    const int64_t wspan = (int64_t)W + 2LL * pw - (int64_t)dw * (S - 1) - 1;
    if (hspan < 0 || wspan < 0) return IGC_ERR_INVALID_VALUE;
    const int64_t P = hspan / sh + 1, Q = wspan / sw + 1;
    const int64_t Mg = (int64_t)N * P * Q, Ng = K, Kg = (int64_t)R * S * C;
    const Plan pl = pick(tune, fp16, true, true, true, Mg, Ng, Kg);
    if (!pl.valid) return IGC_ERR_INVALID_VALUE;
    const Instance* inst = pl.inst;
    if (!inst) return IGC_ERR_UNSUPPORTED;
    if (Mg == 0 || Ng == 0) return IGC_OK;
    if (!x || !w || !y) return IGC_ERR_INVALID_VALUE;
    if (C % 8 != 0) return IGC_ERR_MISALIGNED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return IGC_ERR_MISALIGNED;
    if ((int64_t)N * H * W * C * 2 >= 0x7fffffffLL) return IGC_ERR_UNSUPPORTED;
    if ((inst->bn * Kg + inst->bk) * 2 >= 0x7fffffffLL) return IGC_ERR_UNSUPPORTED;
    // K indices (with the padding tiles past K) must stay below 2^31
    if (P > 0x7fff || Q > 0x7fff || Kg > 0x7fff0000) return IGC_ERR_UNSUPPORTED;

    Params p = {};
    p.A = x;
    p.B = w;
    p.C = y;
    p.M = Mg;
    p.N = Ng;
    p.K = Kg;
    p.lda = 0;
    p.ldb = Kg;
    p.ldc = K;
    p.tiles_m = (int)((Mg + inst->bm - 1) / inst->bm);
    p.tiles_n = (int)((Ng + inst->bn - 1) / inst->bn);
    if ((Mg + inst->bm - 1) / inst->bm > 0x7fffffff) return IGC_ERR_UNSUPPORTED;
    p.out_kind = (int)yt;
    p.group_m = IGC_GROUP_M;
    p.k_ragged8 = 0;  // C % 8 == 0
    p.vec_ok = (K % 8) == 0;  // NPQK rows are K elements: vector stores need 16-byte rows
    p.H = H;
    p.W = W;
    p.Cin = C;
    p.R = R;
    p.S = S;
    p.P = (int)P;
    p.Q = (int)Q;
    p.sh = sh;
    p.sw = sw;
    p.ph = ph;
    p.pw = pw;
    p.dh = dh;
    p.dw = dw;
    p.conv_uniform = (C % inst->bk) == 0;
    p.conv_masks = R <= 16 && S <= 16;
    p.tpt = p.conv_uniform ? C / inst->bk : 1;
    p.cin_magic = fastdiv_magic((uint32_t)C);
    p.s_magic = fastdiv_magic((uint32_t)S);
    p.tpt_magic = fastdiv_magic((uint32_t)p.tpt);
    return launch(pl, p, stream);
}

}  // namespace igc

using namespace igc;

extern "C" {

igc_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la, const void* B,
                       int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type, igc_stream_t stream) {
    return gemm_any(false, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, nullptr, (hipStream_t)stream);
}

igc_status_t gemm_fp16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la, const void* B,
                       int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type, igc_stream_t stream) {
    return gemm_any(true, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, nullptr, (hipStream_t)stream);
}

igc_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la,
                          const void* B, int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t* tune, igc_stream_t stream) {
    return gemm_any(false, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune, (hipStream_t)stream);
}

igc_status_t gemm_fp16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la,
                          const void* B, int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t* tune, igc_stream_t stream) {
    return gemm_any(true, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h, int stride_w,
                                       int pad_h, int pad_w, int dil_h, int dil_w, const void* x, const void* w,
                                       void* y, igc_out_t y_type, igc_stream_t stream) {
    return conv_any(false, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y, y_type,
                    nullptr, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                            int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                            const void* x, const void* w, void* y, igc_out_t y_type,
                                            igc_stream_t stream) {
    return conv_any(true, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y, y_type,
                    nullptr, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                          int stride_w, int pad_h, int pad_w, int dil_h, int dil_w, const void* x,
                                          const void* w, void* y, igc_out_t y_type, int fp16,
                                          const igc_tune_t* tune, igc_stream_t stream) {
    return conv_any(fp16 != 0, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                    y_type, tune, (hipStream_t)stream);
}

int igc_tune_supported(const igc_tune_t* tune) {
    if (!tune) return 0;
    return find_instance(*tune, false, true, false, false) != nullptr;
}

int igc_default_tune(int64_t M, int64_t N, int64_t K, int conv, igc_tune_t* out) {
    if (!out || M < 0 || N < 0 || K < 0) return 0;
    *out = default_tune(M, N, K, conv != 0);
    return 1;
}

int igc_tune_count(void) { return num_tunes(); }

int igc_tune_get(int i, igc_tune_t* out) {
    if (!out || i < 0 || i >= num_tunes()) return 0;
    *out = tune_at(i);
    return 1;
}

int64_t igc_tune_lds_bytes(const igc_tune_t* tune) {
    if (!tune) return 0;
    const Instance* inst = find_instance(*tune, false, true, false, false);
    return inst ? inst->lds_bytes : 0;
}

const char* igc_status_string(igc_status_t status) {
    switch (status) {
        case IGC_OK: return "IGC_OK";
        case IGC_ERR_INVALID_VALUE: return "IGC_ERR_INVALID_VALUE: invalid size, leading dimension, enum or pointer";
        case IGC_ERR_MISALIGNED: return "IGC_ERR_MISALIGNED: pointer or leading dimension not 16-byte aligned";
        case IGC_ERR_UNSUPPORTED: return "IGC_ERR_UNSUPPORTED: configuration not compiled or operand too large";
        case IGC_ERR_HIP: return "IGC_ERR_HIP: the HIP runtime failed to launch the kernel";
    }
    return "unknown igc_status_t";
}

int igc_lds_chunk(int k_contiguous, int chunks_per_row, int row, int logical_chunk) {
    if (row < 0 || logical_chunk < 0 || logical_chunk >= chunks_per_row) return -1;
    if (k_contiguous) {
        if (chunks_per_row == 8) return logical_chunk ^ swz_k<8>(row);
        if (chunks_per_row == 4) return logical_chunk ^ swz_k<4>(row);
        return -1;
    }
    if (chunks_per_row < 16 || chunks_per_row % 16 != 0) return -1;
    return logical_chunk ^ swz_mn(row);
}

int igc_ring_schedule(int D, int half, int KT, int* ev, int cap) {
    if (D < 1 || D > 8 || half < 0 || half > 1 || (half && D < 2) || KT < 0 || cap < 0 || (cap > 0 && !ev))
        return -1;
    const int U = Ring::units(D, half);
    int n = 0;
    auto emit = [&](int kind, int tile, int op, int x) {
        if (n < cap) {
            ev[4 * n] = kind;
            ev[4 * n + 1] = tile;
            ev[4 * n + 2] = op;
            ev[4 * n + 3] = x;
        }
        ++n;
    };
    enum { ISSUE = 0, WAIT = 1, READ = 2, BARRIER = 3 };
    auto issue_unit = [&](int s) { emit(ISSUE, s / 2, s % 2, Ring::slot_of(U, s)); };
    auto read_tile = [&](int t) {
        emit(READ, t, 0, Ring::slot_of(U, 2 * t));
        emit(READ, t, 1, Ring::slot_of(U, 2 * t + 1));
    };
    // the K loop is padded to whole ring periods with zero-filled tiles
    const int P = Ring::period(U);
    const int KTp = (KT + P - 1) / P * P;
    if (Ring::spread(U)) {
        for (int s = 0; s < U - 2; ++s) issue_unit(s);
        emit(WAIT, 0, -1, Ring::wait_units(U));
        if (KTp > 0)
            read_tile(0);
        else
            emit(BARRIER, 0, -1, 0);  // K == 0: the kernel reads zeros it never uses
        for (int t = 0; t < KTp; ++t) {
            issue_unit(2 * t + U - 2);  // both spread over tile t's k-steps
            issue_unit(2 * t + U - 1);
            if (t + 1 < KTp) {
                emit(WAIT, t + 1, -1, Ring::wait_units(U));
                read_tile(t + 1);
            } else {
                emit(BARRIER, t, -1, 0);
            }
        }
    } else if (D >= 2) {
        for (int t = 0; t < D; ++t)
            if (t < KTp) {
                issue_unit(2 * t);
                issue_unit(2 * t + 1);
            }
        if (KTp > 0) {
            emit(WAIT, 0, -1, 2 * Ring::inflight_after(D, KTp, 0));
            read_tile(0);
        }
        for (int t = 0; t < KTp; ++t) {
            if (t + 1 < KTp) {
                emit(WAIT, t + 1, -1, 2 * Ring::inflight_after(D, KTp, t + 1));
                if (t + D < KTp) {
                    issue_unit(2 * (t + D));
                    issue_unit(2 * (t + D) + 1);
                }
                read_tile(t + 1);
            } else {
                emit(BARRIER, t, -1, 0);  // drained; the kernel's trailing read is of no tile
            }
        }
    } else {
        if (KT > 0) {
            issue_unit(0);
            issue_unit(1);
            emit(WAIT, 0, -1, 0);
            read_tile(0);
        }
        for (int t = 0; t < KT; ++t) {
            emit(BARRIER, t, -1, 0);
            if (t + 1 < KT) {
                issue_unit(2 * (t + 1));
                issue_unit(2 * (t + 1) + 1);
                emit(WAIT, t + 1, -1, 0);
                read_tile(t + 1);
            } else {
                emit(BARRIER, t, -1, 0);
            }
        }
    }
    return n;
}

}  // extern "C"
