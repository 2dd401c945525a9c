/*
 * igc.h -- C ABI of libigc: a software-pipelined bf16/fp16 GEMM with fp32
 * accumulation, and the same mainloop run as implicit-GEMM (im2col) NHWC
 * convolutions (forward, data gradient, filter gradient), for AMD Instinct
 * MI355X (gfx950).
 *
 * What is computed follows the "B200 TMA Pipeline Designer" page (section
 * "E -- Executable steps": a tiled matrix product fed by a ring of PIPE_DEPTH
 * shared-memory stages under ready/free synchronisation, with a prologue /
 * steady-state / epilogue timeline) and the "two free pipeline stages" note
 * (section "The atom changes the fragment": the same pipelined mainloop
 * driving an implicit-GEMM convolution with IM2COL operand loads).  The pages'
 * NVIDIA mechanisms (TMA descriptors, mbarriers, elected issuer lanes, 2-SM
 * atoms) are not used; the library uses gfx950 direct-to-LDS buffer loads,
 * s_waitcnt / s_barrier (or LDS counters) and MFMA.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   never frees or retains them; calls are thread-safe.
 * - Each call only validates its arguments and enqueues work on `stream` (a
 *   hipStream_t; NULL = the default stream), which must belong to the current
 *   device.  It returns before the GPU finishes; synchronise the stream to
 *   observe the result.
 * - Workspace.  A call whose schedule splits K (k_splits > 1, or stream-K)
 *   needs an fp32 workspace of igc_workspace_bytes(...) bytes.  The `_ex`
 *   entry points take it from the caller (`workspace`, 256-byte aligned,
 *   `workspace_bytes` at least that size); the call then allocates nothing.
 *   With workspace == NULL (and always for the entry points without `_ex`)
 *   the library takes it stream-ordered on `stream` from a memory pool it
 *   creates on the current device at the first such call, and releases it
 *   with hipFreeAsync on the same stream; the pool keeps up to 256 MiB of freed
 *   workspace mapped until the process ends (the device's default pool is not
 *   changed).  A schedule that does not split K needs and takes nothing.
 *   Calls that share one workspace must be ordered (one stream).  On a stream
 *   that is being captured into a graph, a call whose schedule needs a
 *   workspace must be given one (or use gemm_bf16_noalloc): the library does
 *   not take one from its pool during capture (IGC_ERR_UNSUPPORTED).
 * - Leading dimensions are in ELEMENTS, not bytes.
 * - Alignment: every tensor base pointer must be 16-byte aligned and every
 *   leading dimension times the element size a multiple of 16 bytes (8
 *   elements for 16-bit types, 4 for fp32).  Otherwise IGC_ERR_MISALIGNED.
 * - Arguments are checked before anything is launched; on any error nothing
 *   is enqueued and the output is untouched.  No exception crosses the ABI.
 * - Outputs must not alias inputs (not checked; the result is undefined).
 * - Results are deterministic: the same inputs and tune give the same bits on
 *   every call (no atomics; a fixed summation order per output element).
 * - Device errors: a stream-K owner waits for the partials of the workgroups
 *   sharing its tile with a bounded poll.  If a wait ever gives up (which a
 *   correct schedule with every workgroup resident never does) the owner
 *   writes its tile as NaN and sets the device's error word, which
 *   igc_take_device_error reads.
 */
#ifndef IGC_H
#define IGC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *igc_stream_t; /* the same type as hipStream_t */

typedef enum {
    IGC_OK = 0,
    IGC_ERR_INVALID_VALUE = 1, /* negative size, leading dimension too small, bad enum, NULL pointer, short workspace */
    IGC_ERR_MISALIGNED = 2,    /* pointer or leading dimension breaks the 16-byte rule; conv channels % 8 != 0 */
    IGC_ERR_UNSUPPORTED = 3,   /* tuning choice not compiled in, or an operand span / index >= 2^31 */
    IGC_ERR_HIP = 4            /* the HIP runtime reported an error when allocating or launching */
} igc_status_t;

typedef enum { IGC_ROW_MAJOR = 0, IGC_COL_MAJOR = 1 } igc_layout_t;

typedef enum { IGC_OUT_F32 = 0, IGC_OUT_BF16 = 1, IGC_OUT_F16 = 2 } igc_out_t;

/* The operation whose GEMM view a workspace or default-tile query is about. */
typedef enum { IGC_OP_GEMM = 0, IGC_OP_CONV_FPROP = 1, IGC_OP_CONV_DGRAD = 2, IGC_OP_CONV_WGRAD = 3 } igc_op_t;

/* Optional tuning.
 *   bm, bn, bk    output tile BM x BN and K tile BK;
 *   pipe_depth    number of LDS stages in the ring ("PIPE_DEPTH" of the B200
 *                 TMA Pipeline Designer page, Executable steps 6 and 7);
 *   waves         wave64s per workgroup (4: one per SIMD; 8: two per SIMD);
 *   mfma          MFMA block edge (32: v_mfma_f32_32x32x16, 16:
 *                 v_mfma_f32_16x16x32; 0 means 32);
 *   half_stage    1: the ring holds one more operand tile (A or B) than
 *                 pipe_depth whole stages (2*pipe_depth + 1 operand slots);
 *   loader_waves  how many waves issue the global->LDS loads (0 or `waves`:
 *                 every wave; 4 of 8: one per SIMD);
 *   k_splits      <= 1: none; S > 1: split K into up to S ranges computed by
 *                 separate workgroups whose fp32 partial tiles a second kernel
 *                 sums in split order;
 *   stream_k      0: none; G > 0: a persistent grid of G workgroups takes
 *                 equal runs of the tiles' K ranges, in units of one ring
 *                 period; a tile shared by several runs is finished by the
 *                 workgroup that computes its last K unit, which adds the fp32
 *                 partials of the others in a fixed order (deterministic).
 *                 Assumes the G workgroups are resident together (G at most
 *                 the CU count, nothing else occupying the device);
 *   ring_sync     0: one workgroup barrier per K tile is both the "ready" and
 *                 the "free" signal; 1: per-slot LDS ready/free counters
 *                 (Executable step 4: every stage has its own ready and free
 *                 signal with one producer side and one consumer side);
 *   sk_hybrid     with stream_k: 1 runs whole tiles in data-parallel rounds
 *                 first and splits only the last, partial round's tiles into
 *                 K runs; 0 splits every tile.
 * k_splits > 1 together with stream_k > 0, stream_k < 0, or sk_hybrid without
 * stream_k is IGC_ERR_INVALID_VALUE.  Only compiled (bm, bn, bk, pipe_depth,
 * waves, mfma, half_stage, loader_waves, ring_sync) combinations are accepted
 * (igc_tune_count / igc_tune_get list them, igc_tune_scope says what each
 * is built for); NULL selects the built-in choice for the shape
 * (igc_default_tune). */
typedef struct {
    int bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves, k_splits, stream_k, ring_sync, sk_hybrid;
} igc_tune_t;

/*
 * GEMM: C = A * B with bf16 inputs, fp32 accumulation, output type `c_type`.
 * The tiled, software-pipelined product of the "B200 TMA Pipeline Designer"
 * page (section "E -- Executable steps", steps 6-8).
 *   A is M x K: IGC_ROW_MAJOR -> A[i*lda + k] (lda >= K);
 *               IGC_COL_MAJOR -> A[k*lda + i] (lda >= M).
 *   B is K x N: IGC_ROW_MAJOR -> B[k*ldb + j] (ldb >= N);
 *               IGC_COL_MAJOR -> B[j*ldb + k] (ldb >= K).
 *   C is M x N row-major: C[i*ldc + j] (ldc >= N), element type per c_type;
 *     fp32 -> bf16/fp16 rounds to nearest-even.
 * K == 0 writes zeros; M == 0 or N == 0 is a no-op returning IGC_OK.
 * Errors: IGC_ERR_INVALID_VALUE for negative sizes, bad enums, NULL pointers or
 * leading dimensions below the minimum; IGC_ERR_MISALIGNED; IGC_ERR_UNSUPPORTED
 * when one tile's rows span 2^31 bytes or more; IGC_ERR_HIP.
 */
igc_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                       const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                       igc_stream_t stream);

/* The same contract with IEEE binary16 (fp16) inputs. */
igc_status_t gemm_fp16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                       const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                       igc_stream_t stream);

/* gemm_bf16 / gemm_fp16 with an explicit tile, pipeline depth and schedule
 * (tune == NULL: the built-in choice) and a caller-owned workspace (see the
 * conventions above; NULL: the library's pool).  A non-NULL workspace shorter
 * than igc_workspace_bytes(IGC_OP_GEMM, M, N, K, tune) or not 256-byte
 * aligned is IGC_ERR_INVALID_VALUE. */
igc_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                          const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t *tune, void *workspace, int64_t workspace_bytes, igc_stream_t stream);
igc_status_t gemm_fp16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                          const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t *tune, void *workspace, int64_t workspace_bytes, igc_stream_t stream);

/*
 * Convolutions.  Shared geometry: N images of H x W pixels with C channels,
 * K filters of R x S taps, strides (stride_h, stride_w) >= 1, zero padding
 * (pad_h, pad_w) >= 0, dilations (dil_h, dil_w) >= 1, and the output size
 *   P = (H + 2*pad_h - dil_h*(R-1) - 1)/stride_h + 1,
 *   Q = (W + 2*pad_w - dil_w*(S-1) - 1)/stride_w + 1   (both must be >= 1).
 * Layouts: x NHWC (N*H*W*C elements), w KRSC (K*R*S*C), y NPQK (N*P*Q*K), all
 * dense.  Requirements: H, W, C, R, S >= 1 and N, K >= 0, else
 * IGC_ERR_INVALID_VALUE (an empty output is a no-op; an empty sum -- the data
 * gradient with K = 0, the filter gradient with N = 0 -- writes zeros); C % 8 == 0 (and K % 8 == 0 for the gradients),
 * else IGC_ERR_MISALIGNED; every tensor spanning < 2^31 bytes and every GEMM
 * dimension and index below 2^31, else IGC_ERR_UNSUPPORTED.
 */

/*
 * Forward convolution (cross-correlation) as an implicit GEMM, bf16 inputs,
 * fp32 accumulation: the convolution that the "two free pipeline stages" note
 * runs through the pipelined mainloop with IM2COL operand loads (section "The
 * atom changes the fragment"):
 *   y[n][p][q][k] = sum_{r<R, s<S, c<C} x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c] * w[k][r][s][c]
 * with taps outside the H x W image contributing nothing.  y has type y_type.
 * GEMM view (for igc_workspace_bytes / igc_default_tune): M = N*P*Q,
 * N_gemm = K, K_gemm = R*S*C.
 */
igc_status_t conv2d_nhwc_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                       int stride_w, int pad_h, int pad_w, int dil_h, int dil_w, const void *x,
                                       const void *w, void *y, igc_out_t y_type, igc_stream_t stream);
/* The same contract with IEEE binary16 (fp16) x and w. */
igc_status_t conv2d_nhwc_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                            int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                            const void *x, const void *w, void *y, igc_out_t y_type,
                                            igc_stream_t stream);
/* With an explicit tune and a caller-owned workspace (as gemm_bf16_ex). */
igc_status_t conv2d_nhwc_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                          int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                          const void *x, const void *w, void *y, igc_out_t y_type,
                                          const igc_tune_t *tune, void *workspace, int64_t workspace_bytes,
                                          igc_stream_t stream);
igc_status_t conv2d_nhwc_implicit_gemm_fp16_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                               int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                               const void *x, const void *w, void *y, igc_out_t y_type,
                                               const igc_tune_t *tune, void *workspace, int64_t workspace_bytes,
                                               igc_stream_t stream);

/*
 * Data gradient of the forward convolution above, as an implicit GEMM on the
 * same mainloop: with dy (NPQK, the gradient of y) and w (KRSC),
 *   dx[n][h][w][c] = sum over (r, s, k) of dy[n][p][q][k] * w[k][r][s][c]
 * over the filter taps whose forward read lands on (h, w), i.e.
 * p*sh - ph + r*dh = h and q*sw - pw + s*dw = w for integers 0 <= p < P,
 * 0 <= q < Q.  dx (NHWC) has type dx_type and is fully written (pixels no tap
 * reaches get 0).  The pages run only the forward pass through the mainloop;
 * this is its adjoint in x, the other operand iterator the same mainloop
 * serves.  GEMM view: M = N*H*W, N_gemm = C, K_gemm = R*S*K.  A unit stride
 * and R, S <= 16 use per-pixel tap masks; other strides test each tap's
 * landing position for divisibility by the stride.
 */
igc_status_t conv2d_nhwc_dgrad_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                             int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                             const void *dy, const void *w, void *dx, igc_out_t dx_type,
                                             igc_stream_t stream);
igc_status_t conv2d_nhwc_dgrad_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                  int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                  const void *dy, const void *w, void *dx, igc_out_t dx_type,
                                                  igc_stream_t stream);
igc_status_t conv2d_nhwc_dgrad_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                const void *dy, const void *w, void *dx, igc_out_t dx_type,
                                                const igc_tune_t *tune, void *workspace, int64_t workspace_bytes,
                                                igc_stream_t stream);
igc_status_t conv2d_nhwc_dgrad_implicit_gemm_fp16_ex(int N, int H, int W, int C, int K, int R, int S,
                                                     int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                                                     int dil_w, const void *dy, const void *w, void *dx,
                                                     igc_out_t dx_type, const igc_tune_t *tune, void *workspace,
                                                     int64_t workspace_bytes, igc_stream_t stream);

/*
 * Filter gradient of the forward convolution above, as an implicit GEMM on
 * the same mainloop: with x (NHWC) and dy (NPQK),
 *   dw[k][r][s][c] = sum over (n, p, q) of dy[n][p][q][k] * x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c]
 * with taps outside the image contributing nothing; dw (KRSC) has type
 * dw_type.  The adjoint of the forward convolution in w.  GEMM view:
 * M = K, N_gemm = R*S*C, K_gemm = N*P*Q (deep: the default schedule splits
 * it over the CUs).
 */
igc_status_t conv2d_nhwc_wgrad_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                             int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                             const void *x, const void *dy, void *dw, igc_out_t dw_type,
                                             igc_stream_t stream);
igc_status_t conv2d_nhwc_wgrad_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                  int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                  const void *x, const void *dy, void *dw, igc_out_t dw_type,
                                                  igc_stream_t stream);
igc_status_t conv2d_nhwc_wgrad_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                                int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                                const void *x, const void *dy, void *dw, igc_out_t dw_type,
                                                const igc_tune_t *tune, void *workspace, int64_t workspace_bytes,
                                                igc_stream_t stream);
igc_status_t conv2d_nhwc_wgrad_implicit_gemm_fp16_ex(int N, int H, int W, int C, int K, int R, int S,
                                                     int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                                                     int dil_w, const void *x, const void *dy, void *dw,
                                                     igc_out_t dw_type, const igc_tune_t *tune, void *workspace,
                                                     int64_t workspace_bytes, igc_stream_t stream);

/* gemm_bf16 for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the built-in
 * schedule, with its workspace (K-split or stream-K partial tiles and flags)
 * in a library-owned device array of 16 MiB + 4 KiB that each GPU holds until
 * the process ends.  The call allocates nothing.  When the built-in schedule's
 * workspace fits the array it runs that schedule and gives the same bits as
 * gemm_bf16; otherwise (a K split of 256 x 128 tiles, e.g. 1024 x 1024 x 65536)
 * it runs 128 x 128 stream-K over 256 workgroups, whose workspace always fits,
 * with a different summation order.  Calls that overlap on one GPU share the
 * array and race: order them (one stream).  IGC_ERR_HIP if the array cannot
 * be located on the current device; otherwise as gemm_bf16. */
igc_status_t gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                               const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                               igc_stream_t stream);

/* Workspace bytes a call needs for operation `op` with GEMM view M x N x K
 * (see each operation above) under `tune` (NULL: the built-in choice): 0 when
 * the schedule does not split K.  Returns -1 for negative sizes, a bad op or
 * an invalid tune. */
int64_t igc_workspace_bytes(igc_op_t op, int64_t M, int64_t N, int64_t K, const igc_tune_t *tune);

/* 1 if (bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves, ring_sync) is a compiled
 * configuration (for the bf16 GEMM with row-major A at least), else 0. */
int igc_tune_supported(const igc_tune_t *tune);

/* The configuration the library picks for operation `op` with GEMM view
 * M x N x K when no tune is given; 1 on success. */
int igc_default_tune(igc_op_t op, int64_t M, int64_t N, int64_t K, igc_tune_t *out);

/* Number of compiled configurations; igc_tune_get(i, &t) fills t for i in [0, count).
 * igc_tune_scope(i) is a bit mask of what configuration i is built for: IGC_SCOPE_ALL (every input type,
 * operand layout, operation and loop variant; without it only the bf16 and fp16 GEMM with row-major A and
 * K % 8 == 0, and the bf16 forward convolution with whole filter taps per K tile and filters of at most
 * 16 x 16 -- other calls are IGC_ERR_UNSUPPORTED), IGC_SCOPE_STREAM_K (stream-K schedules; without it
 * a tune with stream_k > 0 is IGC_ERR_UNSUPPORTED) and IGC_SCOPE_CONV_FPROP (the bf16 and fp16 forward
 * convolution with every loop variant, besides the GEMMs with row-major A); 0 for an index out of range. */
enum { IGC_SCOPE_ALL = 1, IGC_SCOPE_STREAM_K = 2, IGC_SCOPE_CONV_FPROP = 4 };
int igc_tune_count(void);
int igc_tune_get(int i, igc_tune_t *out);
int igc_tune_scope(int i);

/* LDS bytes one workgroup of the given configuration uses (0 if not compiled). */
int64_t igc_tune_lds_bytes(const igc_tune_t *tune);

/* Static text for a status code (never NULL). */
const char *igc_status_string(igc_status_t status);

/* Reads the current device's error word into *word (0: no stream-K wait has
 * given up since the last call) and clears it.  Synchronous: it waits for the
 * device's outstanding work.  IGC_ERR_INVALID_VALUE for NULL, IGC_ERR_HIP if
 * the copy fails. */
igc_status_t igc_take_device_error(int *word);

/* Test hook: for later stream-K launches in this process, poll a partial's
 * flag at most `spin_limit` times (<= 0: the built-in bound, about a second of
 * polling) and never raise the flag of workgroup `drop_workgroup` (-1: raise
 * all).  Lets a test make the bounded wait give up while every kernel still
 * exits normally. */
void igc_debug_stream_k(int spin_limit, int drop_workgroup);

/* Number of workspaces the library has taken from its own pool in this
 * process (a call given a workspace, or needing none, adds nothing). */
int64_t igc_pool_allocations(void);

/*
 * Ring schedule of the mainloop, for inspection and testing on the host.
 * The LDS ring holds U = 2*pipe_depth + half_stage operand slots; the K loop
 * consumes units, unit 2t being the A tile and unit 2t+1 the B tile of K tile
 * t, and unit s always lives in slot s % U.  For a K loop of `k_tiles` tiles,
 * writes up to `cap` events into `events` as int quadruples
 * (kind, tile, operand, x):
 *   kind 0 = issue the loads of operand `operand` (0: A, 1: B) of `tile` into
 *            slot x,
 *   kind 1 = wait until both operands of `tile` have landed (each wave waits
 *            on its own loads, then the workgroup barrier runs); x is how many
 *            newer units the wave's s_waitcnt vmcnt lets stay in flight
 *            (operand is -1),
 *   kind 2 = read operand `operand` of `tile` from slot x (fragment loads,
 *            then MFMAs),
 *   kind 3 = workgroup barrier only (pipe_depth 1 frees its single stage with
 *            it; every schedule ends with one once nothing is left in flight).
 * Rings of up to four slots pad the K loop to a whole number of ring periods
 * (U/2 tiles; no padding for pipe_depth 1) with tiles whose loads are all out
 * of range: they land as zeros and add nothing, so tiles up to that padded
 * count appear.  Rings of five or more slots run exactly k_tiles tiles: they
 * issue units 0..U-3 up front and, during each tile t, units 2t+U-2 and
 * 2t+U-1 (interleaved with t's MFMAs) into the two slots the last barrier
 * freed; units past k_tiles are issued out of range and never read.  Two-stage rings issue tile
 * t+2 right after the barrier that frees tile t.  Each wave drains its own
 * LDS reads before every barrier, so a barrier after a unit's reads frees its
 * slot.  (With ring_sync 1 the barrier of a wait event is replaced by the
 * slot's ready counter, and a slot is refilled once its free counter shows
 * every wave done with it; the order of issues, waits and reads is the same.)
 * Returns the number of events (which may exceed cap), or -1 on bad input
 * (pipe_depth outside 1..8, half_stage not 0/1 or with pipe_depth 1, negative
 * k_tiles or cap).  The kernels' loops are written to follow this sequence;
 * the GPU tests' K-chain tags check that they do.
 */
int igc_ring_schedule(int pipe_depth, int half_stage, int k_tiles, int *events, int cap);

/*
 * LDS swizzle of the operand tiles, for inspection and testing on the host.
 * Operand tiles live in LDS as rows of 16-byte chunks; the chunk holding
 * logical chunk `logical_chunk` of row `row` is stored at the returned
 * physical chunk of the same row.  k_contiguous = 1: rows of the K tile
 * (chunks_per_row = BK/8, 8 or 4); 0: rows of BM or BN elements read with the
 * transposing LDS load (chunks_per_row 8 or a multiple of 16).  Returns -1 for an
 * unsupported geometry.  These are the maps the kernels use.
 */
int igc_lds_chunk(int k_contiguous, int chunks_per_row, int row, int logical_chunk);

/*
 * LDS swizzle of the output epilogue's staged rows, for inspection and
 * testing on the host.  A wave stages its 16-bit output sub-tile in LDS as
 * rows of slots_per_row 8-byte slots (16: 128-byte rows, 32: 256-byte rows);
 * logical slot `slot` of row `row` is stored at the returned physical slot of
 * the same row.  Returns -1 for a negative row, a slot outside the row or
 * another row width.  This is the map the kernels use.
 */
int igc_stage_slot(int row, int slot, int slots_per_row);

#ifdef __cplusplus
}
#endif

#endif /* IGC_H */
