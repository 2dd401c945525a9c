// igc_lib.hip -- C ABI of libigc: argument checks, instance selection, launch.
//
// Every entry point validates its arguments completely before it enqueues
// anything, then launches its kernels on the caller's stream and returns.  The
// only memory it may allocate is the fp32 workspace of a K split or a stream-K
// schedule, and only when the caller passes none: then it is taken
// stream-ordered from a pool the library keeps per device.
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

// The device error word: a stream-K owner whose bounded wait gives up sets it
// to 1 (and writes its tile as NaN).  Each GPU holds its own copy.
static __device__ __align__(256) int g_err_word;

// Workspace of gemm_bf16_noalloc, for callers that cannot allocate: room for
// stream-K over 256 workgroups of 128 x 128 fp32 partials (16 MiB + 1 KiB) and
// for a 2-way split of at most 128 tiles of 128 x 128 (16 MiB); a built-in
// schedule that needs more runs as that stream-K instead.  Each GPU the library runs on holds its
// own copy until the process ends; calls that overlap on one GPU share it and
// race.
constexpr int64_t kScratchBytes = (16ll << 20) + 4096;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace igc {

constexpr int kMaxDevices = 64;

static bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Per-device addresses of the library's device variables, looked up once per
// device with that device current.  nullptr if the lookup failed.
static int* err_word_ptr() {
    static std::mutex mu;
    static int* ptrs[kMaxDevices];
    static bool tried[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!tried[dev]) {
        tried[dev] = true;
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_err_word)) == hipSuccess) ptrs[dev] = (int*)ptr;
        (void)hipGetLastError();
    }
    return ptrs[dev];
}

// The current device's copy of `scratch`, looked up once per device with that
// device current (the array's name is only a host-side stand-in); nullptr if
// the lookup failed.
static void* scratch_ptr() {
    static std::mutex mu;
    static void* ptrs[kMaxDevices];
    static bool tried[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!tried[dev]) {
        tried[dev] = true;
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) ptrs[dev] = ptr;
        (void)hipGetLastError();
    }
    return ptrs[dev];
}

// Workspaces the caller does not provide come from a stream-ordered memory
// pool of the library's own, one per device, which keeps up to
// kPoolKeepBytes of freed memory mapped for the next call.  (A pool that
// returns its memory at every synchronisation, the default pool's behaviour,
// remaps the workspace on each call: 8-20 us per call for workspaces of 16-64
// MB.)  The default pool is left untouched.
constexpr uint64_t kPoolKeepBytes = 256ull << 20;
static std::atomic<int64_t> g_pool_allocations{0};

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
    if (e != hipSuccess) return nullptr;
    g_pool_allocations.fetch_add(1, std::memory_order_relaxed);
    return ptr;
}

// True if `stream` is being captured into a graph.  A workspace the library
// would take from its pool during capture would become a memory node of the
// caller's graph, allocated from the library's own pool; that use is refused
// (the caller passes a workspace, or calls gemm_bf16_noalloc), since it has
// not been shown to work on this runtime.
static bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st != hipStreamCaptureStatusNone;
}

// Test hooks for the stream-K bounded wait (igc_debug_stream_k).
constexpr int kDefaultSpinLimit = 1 << 20;  // about a second of polling
static std::atomic<int> g_sk_spin_limit{0};
static std::atomic<int> g_sk_drop{-1};

static int out_size(igc_out_t t) { return t == IGC_OUT_F32 ? 4 : 2; }

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct Plan {
    const Instance* inst = nullptr;
    igc_tune_t tune = {};
    bool valid = true;
};

// The tile configuration and schedule for one call: an explicit tune is taken
// as is; otherwise the built-in choice for the operation and shape.
static Plan pick(const igc_tune_t* tune, bool fp16, bool a_kc, bool b_kc, int op, int64_t M, int64_t N, int64_t K) {
    Plan pl;
    pl.tune = tune ? *tune : default_tune(M, N, K, op);
    const igc_tune_t& t = pl.tune;
    pl.inst = find_instance(t, fp16, a_kc, b_kc, op);
    pl.valid = t.stream_k >= 0 && !(t.k_splits > 1 && t.stream_k > 0) && (t.sk_hybrid == 0 || t.sk_hybrid == 1) &&
               !(t.sk_hybrid && t.stream_k <= 0);
    return pl;
}

// How a plan splits the work of an M x N x K view, and the workspace it needs.
struct Layout {
    int64_t tiles = 0;
    // stream-K
    int G = 0;            // persistent workgroups (0: no stream-K)
    int64_t UT = 0;       // K units (ring periods) per tile
    int64_t dp_tiles = 0; // tiles run whole in data-parallel rounds first
    // split-K
    int S = 1;
    int64_t per = 0;      // K per split
    int64_t ldws = 0;
    // workspace layout
    int64_t part_bytes = 0, flag_off = 0, bytes = 0;
};

static Layout layout_of(const Plan& pl, int64_t M, int64_t N, int64_t K) {
    Layout L;
    const Instance* inst = pl.inst;
    L.tiles = ((M + inst->bm - 1) / inst->bm) * ((N + inst->bn - 1) / inst->bn);
    if (L.tiles <= 0) return L;
    const int64_t unit = (int64_t)inst->bk * Ring::period(Ring::units(inst->d, inst->half));
    if (pl.tune.stream_k > 0 && K > 0) {
        const int64_t G0 = pl.tune.stream_k;
        L.UT = (K + unit - 1) / unit;
        L.dp_tiles = pl.tune.sk_hybrid ? L.tiles - L.tiles % G0 : 0;
        const int64_t total = (L.tiles - L.dp_tiles) * L.UT;
        L.G = (int)(L.dp_tiles > 0 ? G0 : (G0 < total ? G0 : total));
        // partial tiles (one slot per workgroup) and one flag per workgroup
        if (total > 0) {
            L.part_bytes = round_up((int64_t)L.G * inst->bm * inst->bn * 4, 256);
            L.flag_off = L.part_bytes;
            L.bytes = L.part_bytes + round_up((int64_t)L.G * 4, 256);
        }
        return L;
    }
    if (pl.tune.k_splits > 1 && K > 0) {
        // each split a whole number of ring periods (no padding tiles inside a split)
        L.per = ((K + pl.tune.k_splits - 1) / pl.tune.k_splits + unit - 1) / unit * unit;
        L.S = (int)((K + L.per - 1) / L.per);
        if (L.S > 1) {
            L.ldws = (N + 3) / 4 * 4;
            L.bytes = round_up((int64_t)L.S * M * L.ldws * 4, 256);
        }
    }
    return L;
}

// The loop variant (kernel) a call needs: the convolutions' gathered operand
// uses per-pixel tap masks when the filter fits 16 x 16 (and, for the data
// gradient, the stride is 1), whole taps per K tile when the gathered channel
// count is a multiple of BK; a GEMM with K % 8 != 0 needs the ragged loop.
static int loop_variant(const Params& p, const Instance* inst) {
    if (inst->op == OP_FPROP || inst->op == OP_DGRAD)
        return !p.conv_masks ? CONV_GENERIC : (p.conv_uniform ? UNIFORM_TAP : PLAIN);
    if (inst->op == OP_WGRAD) return PLAIN;
    return p.k_ragged8 ? RAGGED : PLAIN;
}

// Launches the mainloop (and, for a K split, the fixed-order reduction; for
// stream-K, the flag clearing before it).  The workspace is the caller's, or
// taken from the library's pool and released with hipFreeAsync after the work
// is enqueued, so concurrent calls on different streams never share it.
static igc_status_t launch(const Plan& pl, Params p, void* user_ws, int64_t user_ws_bytes, hipStream_t stream) {
    const Instance* inst = pl.inst;
    const Layout L = layout_of(pl, p.M, p.N, p.K);
    if (L.tiles <= 0) return IGC_OK;
    if (L.tiles * L.S > 0x7fffffff) return IGC_ERR_UNSUPPORTED;
    // a configuration built without this loop variant or without stream-K kernels
    if (!(L.G > 0 ? inst->fn_sk : inst->fn)[loop_variant(p, inst)]) return IGC_ERR_UNSUPPORTED;
    if (user_ws && (user_ws_bytes < L.bytes || (reinterpret_cast<uintptr_t>(user_ws) & 255u)))
        return IGC_ERR_INVALID_VALUE;
    int* err = err_word_ptr();
    if (!err) return IGC_ERR_HIP;
    p.err_word = err;
    (void)hipGetLastError();  // launch errors below are ours alone
    char* ws = (char*)user_ws;
    const bool owned = !user_ws && L.bytes > 0;
    if (owned && capturing(stream)) return IGC_ERR_UNSUPPORTED;
    if (owned) {
        ws = (char*)workspace_alloc((size_t)L.bytes, stream);
        if (!ws) return IGC_ERR_HIP;
    }
    hipError_t e = hipSuccess;
    unsigned grid = 0;
    const int v = loop_variant(p, inst);
    const void* fn = L.G > 0 ? inst->fn_sk[v] : inst->fn[v];
    if (L.G > 0) {
        p.sk_grid = L.G;
        p.sk_units = L.UT;
        p.sk_dp_tiles = L.dp_tiles;
        p.sk_ws = (float*)ws;
        p.sk_flags = ws ? (int*)(ws + L.flag_off) : nullptr;
        const int spin = g_sk_spin_limit.load(std::memory_order_relaxed);
        p.sk_spin_limit = spin > 0 ? spin : kDefaultSpinLimit;
        p.sk_drop = g_sk_drop.load(std::memory_order_relaxed);
        p.k_splits = 1;
        p.k_per_split = p.K;
        grid = (unsigned)L.G;
        if (p.sk_flags) e = launch_clear_flags(p.sk_flags, L.G, stream);
    } else {
        p.sk_grid = 0;
        p.k_splits = L.S;
        p.k_per_split = L.S > 1 ? L.per : (p.K > 0 ? p.K : 1);
        if (L.S > 1) {
            p.ldws = L.ldws;
            p.ws_stride = p.M * L.ldws;
            p.ws = (float*)ws;
        }
        grid = (unsigned)(L.tiles * L.S);
    }
    if (e == hipSuccess) {
        Params arg = p;
        void* args[] = {&arg};
        e = hipLaunchKernel(fn, dim3(grid), dim3(64 * inst->waves), args, 0, stream);
    }
    if (e == hipSuccess && L.G == 0 && L.S > 1)
        e = launch_split_reduce(p.ws, L.S, p.ws_stride, p.M, p.N, p.ldws, p.C, p.ldc, p.out_kind, stream);
    if (owned) (void)hipFreeAsync(ws, stream);
    if (e != hipSuccess) return IGC_ERR_HIP;
    return hipGetLastError() == hipSuccess ? IGC_OK : IGC_ERR_HIP;
}

static igc_status_t gemm_any(bool fp16, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             igc_layout_t la, const void* B, int64_t ldb, igc_layout_t lb, void* C, int64_t ldc,
                             igc_out_t ct, const igc_tune_t* tune, void* ws, int64_t ws_bytes, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0) return IGC_ERR_INVALID_VALUE;
    if ((la != IGC_ROW_MAJOR && la != IGC_COL_MAJOR) || (lb != IGC_ROW_MAJOR && lb != IGC_COL_MAJOR))
        return IGC_ERR_INVALID_VALUE;
    if (ct != IGC_OUT_F32 && ct != IGC_OUT_BF16 && ct != IGC_OUT_F16) return IGC_ERR_INVALID_VALUE;
    const bool a_kc = la == IGC_ROW_MAJOR, b_kc = lb == IGC_COL_MAJOR;
    const Plan pl = pick(tune, fp16, a_kc, b_kc, OP_GEMM, M, N, K);
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
    if ((M + inst->bm - 1) / inst->bm > 0x7fffffff || (N + inst->bn - 1) / inst->bn > 0x7fffffff)
        return IGC_ERR_UNSUPPORTED;

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
    p.out_kind = (int)ct;
    p.group_m = IGC_GROUP_M;
    p.k_ragged8 = (K % 8) != 0;
    p.vec_ok = 1;
    return launch(pl, p, ws, ws_bytes, stream);
}

// The GEMM view (M x N x K) of a convolution operation.
static void conv_view(int op, int64_t N, int64_t C, int64_t K, int64_t R, int64_t S, int64_t H, int64_t W, int64_t P,
                      int64_t Q, int64_t& Mg, int64_t& Ng, int64_t& Kg) {
    if (op == OP_FPROP) {
        Mg = N * P * Q, Ng = K, Kg = R * S * C;
    } else if (op == OP_DGRAD) {
        Mg = N * H * W, Ng = C, Kg = R * S * K;
    } else {
        Mg = K, Ng = R * S * C, Kg = N * P * Q;
    }
}

// in0 / in1 / out: FPROP x, w -> y; DGRAD dy, w -> dx; WGRAD x, dy -> dw.
static igc_status_t conv_any(int op, bool fp16, int N, int H, int W, int C, int K, int R, int S, int sh, int sw,
                             int ph, int pw, int dh, int dw, const void* in0, const void* in1, void* out,
                             igc_out_t ot, const igc_tune_t* tune, void* ws, int64_t ws_bytes, hipStream_t stream) {
    if (N < 0 || K < 0 || H < 1 || W < 1 || C < 1 || R < 1 || S < 1 || sh < 1 || sw < 1 || ph < 0 || pw < 0 ||
        dh < 1 || dw < 1)
        return IGC_ERR_INVALID_VALUE;
    if (ot != IGC_OUT_F32 && ot != IGC_OUT_BF16 && ot != IGC_OUT_F16) return IGC_ERR_INVALID_VALUE;
    const int64_t hspan = (int64_t)H + 2LL * ph - (int64_t)dh * (R - 1) - 1;
    const int64_t wspan = (int64_t)W + 2LL * pw - (int64_t)dw * (S - 1) - 1;
    if (hspan < 0 || wspan < 0) return IGC_ERR_INVALID_VALUE;
    const int64_t P = hspan / sh + 1, Q = wspan / sw + 1;
    int64_t Mg, Ng, Kg;
    conv_view(op, N, C, K, R, S, H, W, P, Q, Mg, Ng, Kg);
    // operand layouts of the views: FPROP A row / B col, DGRAD A row / B row, WGRAD A col / B row
    const bool a_kc = op != OP_WGRAD, b_kc = op == OP_FPROP;
    const Plan pl = pick(tune, fp16, a_kc, b_kc, op, Mg, Ng, Kg);
    if (!pl.valid) return IGC_ERR_INVALID_VALUE;
    const Instance* inst = pl.inst;
    if (!inst) return IGC_ERR_UNSUPPORTED;
    if (Mg == 0 || Ng == 0) return IGC_OK;
    if (!out || (Kg > 0 && (!in0 || !in1))) return IGC_ERR_INVALID_VALUE;  // an empty sum reads no input
    if (C % 8 != 0 || (op != OP_FPROP && K % 8 != 0)) return IGC_ERR_MISALIGNED;
    if (!aligned16(in0) || !aligned16(in1) || !aligned16(out)) return IGC_ERR_MISALIGNED;
    // every tensor, GEMM dimension and (padded) K index below 2^31
    constexpr int64_t kLim = 0x7fffffffLL;
    if ((int64_t)N * H * W * C * 2 >= kLim || (int64_t)N * P * Q * K * 2 >= kLim ||
        (int64_t)K * R * S * C * 2 >= kLim || (int64_t)N * P * Q * 4 >= kLim)
        return IGC_ERR_UNSUPPORTED;
    if (Mg > kLim || Ng > kLim || Kg > 0x7fff0000LL || P > 0x7fff || Q > 0x7fff) return IGC_ERR_UNSUPPORTED;
    if (op == OP_FPROP && (inst->bn * Kg + inst->bk) * 2 >= kLim) return IGC_ERR_UNSUPPORTED;

    Params p = {};
    p.A = op == OP_WGRAD ? in1 : in0;  // WGRAD: A = dy
    p.B = op == OP_WGRAD ? in0 : in1;  //        B = x
    p.C = out;
    p.M = Mg;
    p.N = Ng;
    p.K = Kg;
    p.lda = op == OP_WGRAD ? K : 0;
    p.ldb = op == OP_FPROP ? Kg : (op == OP_DGRAD ? (int64_t)R * S * C : 0);
    p.ldc = Ng;
    p.tiles_m = (int)((Mg + inst->bm - 1) / inst->bm);
    p.tiles_n = (int)((Ng + inst->bn - 1) / inst->bn);
    p.out_kind = (int)ot;
    p.group_m = IGC_GROUP_M;
    p.k_ragged8 = 0;              // channel counts are multiples of 8
    p.vec_ok = (Ng % 8) == 0;     // output rows are Ng elements: vector stores need 16-byte rows
    p.H = H;
    p.W = W;
    p.Cin = C;
    p.Kc = K;
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
    if (op == OP_FPROP) {
        p.gH = H, p.gW = W, p.gC = C, p.rP = (int)P, p.rQ = (int)Q;
        p.rsh = sh, p.rsw = sw, p.roh = -ph, p.row = -pw, p.tdh = dh, p.tdw = dw, p.gsh = 1, p.gsw = 1;
    } else if (op == OP_DGRAD) {
        p.gH = (int)P, p.gW = (int)Q, p.gC = K, p.rP = H, p.rQ = W;
        p.rsh = 1, p.rsw = 1, p.roh = ph, p.row = pw, p.tdh = -dh, p.tdw = -dw, p.gsh = sh, p.gsw = sw;
    }
    if (op != OP_WGRAD) {
        // the gathered operand's byte offsets, window origins and tap offsets
        // included, must stay within a signed 32-bit range
        const int64_t hmax = (int64_t)(p.rP - 1) * p.rsh + p.roh, wmax = (int64_t)(p.rQ - 1) * p.rsw + p.row;
        const int64_t span = ((((int64_t)N * p.gH + hmax + 1) * p.gW + wmax + 1) * p.gC) * 2;
        const int64_t taps = (((int64_t)R * dh * p.gW + (int64_t)S * dw) * p.gC + p.gC) * 2;
        if (span + taps >= kLim || (int64_t)ph * W * C * 2 >= kLim) return IGC_ERR_UNSUPPORTED;
    }
    p.gsh_magic = fastdiv_magic((uint32_t)p.gsh);
    p.gsw_magic = fastdiv_magic((uint32_t)p.gsw);
    p.conv_uniform = p.gC > 0 && (p.gC % inst->bk) == 0;
    p.conv_masks = R <= 16 && S <= 16 && (op != OP_DGRAD || (sh == 1 && sw == 1));
    p.tpt = p.conv_uniform ? p.gC / inst->bk : 1;
    p.cin_magic = fastdiv_magic((uint32_t)(p.gC > 0 ? p.gC : 1));
    p.s_magic = fastdiv_magic((uint32_t)S);
    p.tpt_magic = fastdiv_magic((uint32_t)p.tpt);
    p.q_magic = fastdiv_magic((uint32_t)Q);
    p.pq_magic = fastdiv_magic((uint32_t)(P * Q));
    return launch(pl, p, ws, ws_bytes, stream);
}

}  // namespace igc

using namespace igc;

extern "C" {

igc_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la, const void* B,
                       int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type, igc_stream_t stream) {
    return gemm_any(false, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t gemm_fp16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la, const void* B,
                       int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type, igc_stream_t stream) {
    return gemm_any(true, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la,
                          const void* B, int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t* tune, void* workspace, int64_t workspace_bytes, igc_stream_t stream) {
    return gemm_any(false, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune, workspace, workspace_bytes,
                    (hipStream_t)stream);
}

igc_status_t gemm_fp16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la,
                          const void* B, int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t* tune, void* workspace, int64_t workspace_bytes, igc_stream_t stream) {
    return gemm_any(true, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune, workspace, workspace_bytes,
                    (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h, int stride_w,
                                       int pad_h, int pad_w, int dil_h, int dil_w, const void* x, const void* w,
                                       void* y, igc_out_t y_type, igc_stream_t stream) {
    return conv_any(OP_FPROP, false, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                    y_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                            int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                            const void* x, const void* w, void* y, igc_out_t y_type,
                                            igc_stream_t stream) {
    return conv_any(OP_FPROP, true, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                    y_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                          int stride_w, int pad_h, int pad_w, int dil_h, int dil_w, const void* x,
                                          const void* w, void* y, igc_out_t y_type, const igc_tune_t* tune,
                                          void* workspace, int64_t workspace_bytes, igc_stream_t stream) {
    return conv_any(OP_FPROP, false, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                    y_type, tune, workspace, workspace_bytes, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_implicit_gemm_fp16_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                               int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                               const void* x, const void* w, void* y, igc_out_t y_type,
                                               const igc_tune_t* tune, void* workspace, int64_t workspace_bytes,
                                               igc_stream_t stream) {
    return conv_any(OP_FPROP, true, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                    y_type, tune, workspace, workspace_bytes, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_dgrad_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                             int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                             const void* dy, const void* w, void* dx, igc_out_t dx_type,
                                             igc_stream_t stream) {
    return conv_any(OP_DGRAD, false, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, dy, w, dx,
                    dx_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_dgrad_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                  int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                  const void* dy, const void* w, void* dx, igc_out_t dx_type,
                                                  igc_stream_t stream) {
    return conv_any(OP_DGRAD, true, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, dy, w, dx,
                    dx_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_dgrad_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                const void* dy, const void* w, void* dx, igc_out_t dx_type,
                                                const igc_tune_t* tune, void* workspace, int64_t workspace_bytes,
                                                igc_stream_t stream) {
    return conv_any(OP_DGRAD, false, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, dy, w, dx,
                    dx_type, tune, workspace, workspace_bytes, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_dgrad_implicit_gemm_fp16_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                     int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                     const void* dy, const void* w, void* dx, igc_out_t dx_type,
                                                     const igc_tune_t* tune, void* workspace,
                                                     int64_t workspace_bytes, igc_stream_t stream) {
    return conv_any(OP_DGRAD, true, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, dy, w, dx,
                    dx_type, tune, workspace, workspace_bytes, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_wgrad_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                             int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                             const void* x, const void* dy, void* dw, igc_out_t dw_type,
                                             igc_stream_t stream) {
    return conv_any(OP_WGRAD, false, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, dy, dw,
                    dw_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_wgrad_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                  int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                  const void* x, const void* dy, void* dw, igc_out_t dw_type,
                                                  igc_stream_t stream) {
    return conv_any(OP_WGRAD, true, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, dy, dw,
                    dw_type, nullptr, nullptr, 0, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_wgrad_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                const void* x, const void* dy, void* dw, igc_out_t dw_type,
                                                const igc_tune_t* tune, void* workspace, int64_t workspace_bytes,
                                                igc_stream_t stream) {
    return conv_any(OP_WGRAD, false, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, dy, dw,
                    dw_type, tune, workspace, workspace_bytes, (hipStream_t)stream);
}

igc_status_t conv2d_nhwc_wgrad_implicit_gemm_fp16_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                     int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                     const void* x, const void* dy, void* dw, igc_out_t dw_type,
                                                     const igc_tune_t* tune, void* workspace,
                                                     int64_t workspace_bytes, igc_stream_t stream) {
    return conv_any(OP_WGRAD, true, N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, dy, dw,
                    dw_type, tune, workspace, workspace_bytes, (hipStream_t)stream);
}

igc_status_t gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, igc_layout_t la,
                               const void* B, int64_t ldb, igc_layout_t lb, void* C, int64_t ldc, igc_out_t c_type,
                               igc_stream_t stream) {
    // the built-in schedule, with its workspace in this device's scratch array;
    // when that schedule needs more (a K split of 256 x 128 tiles), 128 x 128
    // stream-K over 256 workgroups, whose workspace always fits
    if (M < 0 || N < 0 || K < 0) return IGC_ERR_INVALID_VALUE;
    const bool a_kc = la == IGC_ROW_MAJOR, b_kc = lb == IGC_COL_MAJOR;
    const Plan pl = pick(nullptr, false, a_kc, b_kc, OP_GEMM, M, N, K);
    const igc_tune_t* tune = nullptr;
    static const igc_tune_t kFits = {128, 128, 64, 4, 8, 16, 0, 4, 1, 256, 0, 0};
    if (pl.inst && layout_of(pl, M, N, K).bytes > kScratchBytes) {
        const Plan alt = pick(&kFits, false, a_kc, b_kc, OP_GEMM, M, N, K);
        if (!alt.inst || layout_of(alt, M, N, K).bytes > kScratchBytes) return IGC_ERR_UNSUPPORTED;
        tune = &kFits;
    }
    void* ws = scratch_ptr();
    if (!ws) return IGC_ERR_HIP;
    return gemm_any(false, M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_type, tune, ws, kScratchBytes,
                    (hipStream_t)stream);
}

int64_t igc_workspace_bytes(igc_op_t op, int64_t M, int64_t N, int64_t K, const igc_tune_t* tune) {
    if (M < 0 || N < 0 || K < 0 || (int)op < 0 || (int)op > 3) return -1;
    // the layouts only select among compiled kernels of one configuration; any compiled one sizes the split
    const bool a_kc = op != IGC_OP_CONV_WGRAD, b_kc = op == IGC_OP_GEMM || op == IGC_OP_CONV_FPROP;
    Plan pl = pick(tune, false, a_kc, b_kc, (int)op, M, N, K);
    if (!pl.inst) pl.inst = find_instance(pl.tune, false, true, false, OP_GEMM);
    if (!pl.valid || !pl.inst) return -1;
    if (M == 0 || N == 0) return 0;
    return layout_of(pl, M, N, K).bytes;
}

int igc_tune_supported(const igc_tune_t* tune) {
    if (!tune) return 0;
    return find_instance(*tune, false, true, false, OP_GEMM) != nullptr;
}

int igc_default_tune(igc_op_t op, int64_t M, int64_t N, int64_t K, igc_tune_t* out) {
    if (!out || M < 0 || N < 0 || K < 0 || (int)op < 0 || (int)op > 3) return 0;
    *out = default_tune(M, N, K, (int)op);
    return 1;
}

int igc_tune_count(void) { return num_tunes(); }

int igc_tune_get(int i, igc_tune_t* out) {
    if (!out || i < 0 || i >= num_tunes()) return 0;
    *out = tune_at(i);
    return 1;
}

int igc_tune_scope(int i) { return (i >= 0 && i < num_tunes()) ? tune_scope(i) : 0; }

int64_t igc_tune_lds_bytes(const igc_tune_t* tune) {
    if (!tune) return 0;
    const Instance* inst = find_instance(*tune, false, true, false, OP_GEMM);
    return inst ? inst->lds_bytes : 0;
}

const char* igc_status_string(igc_status_t status) {
    switch (status) {
        case IGC_OK: return "IGC_OK";
        case IGC_ERR_INVALID_VALUE:
            return "IGC_ERR_INVALID_VALUE: invalid size, leading dimension, enum, pointer or workspace";
        case IGC_ERR_MISALIGNED: return "IGC_ERR_MISALIGNED: pointer or leading dimension not 16-byte aligned";
        case IGC_ERR_UNSUPPORTED: return "IGC_ERR_UNSUPPORTED: configuration not compiled or operand too large";
        case IGC_ERR_HIP: return "IGC_ERR_HIP: the HIP runtime failed to allocate or launch";
    }
    return "unknown igc_status_t";
}

igc_status_t igc_take_device_error(int* word) {
    if (!word) return IGC_ERR_INVALID_VALUE;
    int* err = err_word_ptr();
    if (!err) return IGC_ERR_HIP;
    int v = 0;
    if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&v, err, sizeof v, hipMemcpyDeviceToHost) != hipSuccess)
        return IGC_ERR_HIP;
    const int zero = 0;
    if (hipMemcpy(err, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return IGC_ERR_HIP;
    *word = v;
    return IGC_OK;
}

void igc_debug_stream_k(int spin_limit, int drop_workgroup) {
    g_sk_spin_limit.store(spin_limit > 0 ? spin_limit : 0, std::memory_order_relaxed);
    g_sk_drop.store(drop_workgroup >= 0 ? drop_workgroup : -1, std::memory_order_relaxed);
}

int64_t igc_pool_allocations(void) { return g_pool_allocations.load(std::memory_order_relaxed); }

int igc_lds_chunk(int k_contiguous, int chunks_per_row, int row, int logical_chunk) {
    if (row < 0 || logical_chunk < 0 || logical_chunk >= chunks_per_row) return -1;
    if (k_contiguous) {
        if (chunks_per_row == 8) return logical_chunk ^ swz_k<8>(row);
        if (chunks_per_row == 4) return logical_chunk ^ swz_k<4>(row);
        return -1;
    }
    if (chunks_per_row == 8) return logical_chunk ^ swz_mn<8>(row);
    if (chunks_per_row < 16 || chunks_per_row % 16 != 0) return -1;
    return logical_chunk ^ swz_mn<16>(row);
}

int igc_stage_slot(int row, int slot, int slots_per_row) {
    if (row < 0 || slot < 0 || (slots_per_row != 16 && slots_per_row != 32) || slot >= slots_per_row) return -1;
    return stage_slot(row, slot, slots_per_row);
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
    // two-stage rings pad the K loop to whole ring periods with zero-filled
    // tiles; spread rings run exactly KT tiles (a last, partial period after
    // the loop), and the units their last tiles issue past KT land as zeros
    const int P = Ring::period(U);
    const int KTp = (KT + P - 1) / P * P;
    if (Ring::spread(U)) {
        for (int s = 0; s < U - 2; ++s) issue_unit(s);
        emit(WAIT, 0, -1, Ring::wait_units(U));
        if (KT > 0)
            read_tile(0);
        else
            emit(BARRIER, 0, -1, 0);  // K == 0: the kernel reads zeros it never uses
        for (int t = 0; t < KT; ++t) {
            issue_unit(2 * t + U - 2);  // both spread over tile t's k-steps
            issue_unit(2 * t + U - 1);
            if (t + 1 < KT) {
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
