/*
 * igc.h -- C ABI of libigc: a software-pipelined bf16/fp16 GEMM with fp32
 * accumulation, and the same mainloop run as an implicit-GEMM (im2col) NHWC
 * convolution, for AMD Instinct MI355X (gfx950).
 *
 * What is computed follows the "B200 TMA Pipeline Designer" page ("Executable
 * steps": a tiled matrix product fed by a ring of PIPE_DEPTH shared-memory
 * stages under ready/free synchronisation, with a prologue / steady-state /
 * epilogue timeline) and the "two free pipeline stages" note (section "The atom
 * changes the fragment": the same pipelined mainloop driving an implicit-GEMM
 * convolution with IM2COL operand loads).  The pages' NVIDIA mechanisms (TMA
 * descriptors, mbarriers, elected issuer lanes, 2-SM atoms) are not used; the
 * library uses gfx950 direct-to-LDS buffer loads, s_waitcnt/s_barrier and MFMA.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   never frees or retains them and keeps no per-call state (beyond a
 *   process-wide call counter that tags stream-K flags); calls are
 *   thread-safe.  A call that splits K takes a temporary fp32 workspace
 *   (k_splits * M * N * 4 bytes, N rounded up to 4), and a stream-K call one
 *   of G * BM * BN * 4 bytes plus 8 bytes per workgroup, stream-ordered on
 *   `stream` from a memory pool the library creates on the current device at
 *   its first such call, and releases it with hipFreeAsync on the same stream;
 *   no other call allocates.  The pool keeps up to 256 MiB of freed workspace
 *   mapped for later calls until the process ends (the device's default pool
 *   is not changed).  `stream` must belong to the current device.
 * - Each call only validates its arguments and enqueues work on `stream`
 *   (a hipStream_t; NULL = the default stream).  It returns before the GPU
 *   finishes; synchronise the stream to observe the result.
 * - Leading dimensions are in ELEMENTS, not bytes.
 * - Alignment: every tensor base pointer must be 16-byte aligned and every
 *   leading dimension times the element size must be a multiple of 16 bytes
 *   (8 elements for 16-bit types, 4 for fp32).  Otherwise IGC_ERR_MISALIGNED.
 * - Arguments are checked before anything is launched; on any error nothing
 *   is enqueued and the output is untouched.  No exception crosses the ABI.
 * - Outputs must not alias inputs (not checked; the result is undefined).
 * - Results are deterministic: the same inputs give the same bits on every
 *   call (no atomics; a fixed summation order per output element).
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
    IGC_ERR_INVALID_VALUE = 1, /* negative size, leading dimension too small, bad enum, NULL pointer */
    IGC_ERR_MISALIGNED = 2,    /* pointer or leading dimension breaks the 16-byte rule; conv C % 8 != 0 */
    IGC_ERR_UNSUPPORTED = 3,   /* tuning choice not compiled in, or an operand span >= 2^31 bytes */
    IGC_ERR_HIP = 4            /* the HIP runtime reported an error when launching */
} igc_status_t;

typedef enum { IGC_ROW_MAJOR = 0, IGC_COL_MAJOR = 1 } igc_layout_t;

typedef enum { IGC_OUT_F32 = 0, IGC_OUT_BF16 = 1, IGC_OUT_F16 = 2 } igc_out_t;

/* Optional tuning: output tile BM x BN, K tile BK, PIPE_DEPTH = number of LDS
 * stages in the ring, the number of wave64s per workgroup (4: one per SIMD;
 * 8: two per SIMD), the MFMA block edge (32: v_mfma_f32_32x32x16, 16:
 * v_mfma_f32_16x16x32; 0 means 32), half_stage (1: the ring holds one more
 * operand tile, A or B, than PIPE_DEPTH whole stages, i.e. 2*PIPE_DEPTH+1
 * operand slots), loader_waves (how many of the waves issue the global->LDS
 * loads; 0 or `waves` = every wave, 4 of 8 = one per SIMD), k_splits (<= 1:
 * none; S > 1: split K into up to S ranges
 * computed by separate workgroups whose fp32 partial tiles are summed in
 * split order by a second kernel), and stream_k (0: none; G > 0: a
 * persistent grid of G workgroups takes equal runs of the tiles' K ranges, in
 * units of one ring period; a tile shared by several runs is finished by the
 * workgroup that computes its last K unit, which adds the fp32 partials of
 * the others in a fixed order, so results are deterministic; each flag is
 * raised as the pair (epoch, ~epoch) with a per-call 31-bit epoch, so the
 * workspace is never cleared, and only reused memory that happens to hold
 * exactly that pair where a flag lies could be mistaken for a raised flag).  k_splits > 1
 * together with stream_k > 0, or stream_k < 0, is IGC_ERR_INVALID_VALUE.  Only
 * compiled (bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves)
 * combinations are accepted (see igc_tune_supported); NULL selects the built-in choice for the
 * shape (which splits K when the output has too few tiles to occupy every
 * CU).  Stream-K assumes the G workgroups are dispatched in index order (a
 * workgroup only waits on lower-numbered ones); its wait is bounded, so a
 * violation yields wrong results rather than a hang. */
typedef struct {
    int bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves, k_splits, stream_k;
} igc_tune_t;

/*
 * C = A * B with bf16 inputs, fp32 accumulation, output type `c_type`.
 *   A is M x K: IGC_ROW_MAJOR -> A[i*lda + k] (lda >= K);
 *               IGC_COL_MAJOR -> A[k*lda + i] (lda >= M).
 *   B is K x N: IGC_ROW_MAJOR -> B[k*ldb + j] (ldb >= N);
 *               IGC_COL_MAJOR -> B[j*ldb + k] (ldb >= K).
 *   C is M x N row-major: C[i*ldc + j] (ldc >= N), element type per c_type;
 *     fp32 -> bf16/fp16 rounds to nearest-even.
 * K == 0 writes zeros; M == 0 or N == 0 is a no-op returning IGC_OK.
 */
igc_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                       const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                       igc_stream_t stream);

/* Same contract as gemm_bf16 with IEEE binary16 (fp16) inputs. */
igc_status_t gemm_fp16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                       const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                       igc_stream_t stream);

/* gemm_bf16 / gemm_fp16 with an explicit tile and pipeline depth (NULL = default). */
igc_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                          const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t *tune, igc_stream_t stream);
igc_status_t gemm_fp16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, igc_layout_t la,
                          const void *B, int64_t ldb, igc_layout_t lb, void *C, int64_t ldc, igc_out_t c_type,
                          const igc_tune_t *tune, igc_stream_t stream);

/*
 * Forward 2-D convolution (cross-correlation) as an implicit GEMM, bf16
 * inputs, fp32 accumulation:
 *   y[n][p][q][k] = sum_{r<R, s<S, c<C} x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c] * w[k][r][s][c]
 * with zero padding (taps outside the H x W image contribute nothing).
 *   x: NHWC, dense, N*H*W*C elements (bf16).
 *   w: KRSC, dense, K*R*S*C elements (bf16).
 *   y: NPQK, dense, N*P*Q*K elements of type y_type, where
 *      P = (H + 2*ph - dh*(R-1) - 1)/sh + 1,  Q = (W + 2*pw - dw*(S-1) - 1)/sw + 1.
 * Requirements: N, H, W, C, K, R, S >= 1 (N or K may be 0: no-op), strides and
 * dilations >= 1, pads >= 0, P >= 1 and Q >= 1 (else IGC_ERR_INVALID_VALUE);
 * C % 8 == 0 (else IGC_ERR_MISALIGNED); x must span < 2^31 bytes and
 * R*S*C must not exceed 0x7fff0000 (else IGC_ERR_UNSUPPORTED).  The GEMM view
 * is M = N*P*Q, N_gemm = K, K_gemm = R*S*C.
 */
igc_status_t conv2d_nhwc_implicit_gemm(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                       int stride_w, int pad_h, int pad_w, int dil_h, int dil_w, const void *x,
                                       const void *w, void *y, igc_out_t y_type, igc_stream_t stream);

/* Same contract with IEEE binary16 (fp16) x and w. */
igc_status_t conv2d_nhwc_implicit_gemm_fp16(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                            int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                            const void *x, const void *w, void *y, igc_out_t y_type,
                                            igc_stream_t stream);

/* conv2d_nhwc_implicit_gemm with an explicit tile and pipeline depth (NULL = default);
 * `fp16` selects binary16 inputs instead of bf16. */
igc_status_t conv2d_nhwc_implicit_gemm_ex(int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                          int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                          const void *x, const void *w, void *y, igc_out_t y_type, int fp16,
                                          const igc_tune_t *tune, igc_stream_t stream);

/* 1 if (bm, bn, bk, pipe_depth, waves, mfma, half_stage, loader_waves) is a compiled configuration, else 0. */
int igc_tune_supported(const igc_tune_t *tune);

/* The configuration the library picks for an M x N x K problem (conv != 0: the
 * implicit-GEMM view of a convolution) when no tune is given; 1 on success. */
int igc_default_tune(int64_t M, int64_t N, int64_t K, int conv, igc_tune_t *out);

/* Number of compiled configurations; igc_tune_get(i, &t) fills t for i in [0, count). */
int igc_tune_count(void);
int igc_tune_get(int i, igc_tune_t *out);

/* LDS bytes one workgroup of the given configuration uses (0 if not compiled). */
int64_t igc_tune_lds_bytes(const igc_tune_t *tune);

/* Static text for a status code (never NULL). */
const char *igc_status_string(igc_status_t status);

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
 * The K loop is padded to a whole number of ring periods (U tiles for an odd
 * U, U/2 for an even one; no padding for pipe_depth 1) with tiles whose loads
 * are all out of range: they land as zeros and add nothing, so tiles up to
 * that padded count appear.  Rings of five or more slots issue units 0..U-3
 * up front and, during each tile t, units 2t+U-2 and 2t+U-1 (interleaved with
 * t's MFMAs) into the two slots the last barrier freed; units past the padded
 * count are issued out of range and never read.  Two-stage rings issue tile
 * t+2 right after the barrier that frees tile t.  Each wave drains its own
 * LDS reads before every barrier, so a barrier after a unit's reads frees its
 * slot.  Returns the number of events (which may exceed cap), or -1 on bad
 * input (pipe_depth outside 1..8, half_stage not 0/1 or with pipe_depth 1,
 * negative k_tiles or cap).  This is the exact sequence the kernels execute.
 */
int igc_ring_schedule(int pipe_depth, int half_stage, int k_tiles, int *events, int cap);

/*
 * Measurement probes (not part of the GEMM/convolution path; they bound it).
 *
 * igc_probe_mfma: an MFMA-only stream with the wave tile of the GEMM kernels
 * (128 x 64 per wave with 8 waves, 128 x 128 with 4), `mfma` = 16
 * (v_mfma_f32_16x16x32_bf16) or 32 (v_mfma_f32_32x32x16_bf16), on random
 * normal bf16 operands held in registers, no memory traffic: `grid`
 * workgroups of 64*waves threads each run `iters` iterations of two k-steps of
 * the wave tile, i.e. grid*waves*iters*2*(128*W)*(2*32) flop for wave-tile
 * width W (64 or 128), where each k-step is K = 32 deep for mfma 16 and 16
 * deep for mfma 32.  Writes one float per thread to `sink` (keeps the
 * accumulators live; needs grid*64*waves*4 bytes) and, per workgroup g,
 * clk[2g] = shader-clock cycles and clk[2g+1] = 100 MHz ticks of its run
 * (uint32; needs grid*8 bytes).  Asynchronous on `stream`.
 *
 * igc_probe_dma: the tile loads of the 8192^3 GEMM (A and B row-major bf16
 * 8192 x 8192, 256 x 256 tiles in the GEMM's XCD order, 8 waves, 1024
 * workgroups) into an LDS ring paced by vmcnt with a workgroup barrier per K
 * tile, with no LDS reads or MFMAs.  bk = 16, 32 (4 slots) or 64 (2 slots)
 * sets the K tile, i.e. the length of each A row segment (2*bk bytes);
 * operands = 1 (A only), 2 (B only) or 3 (both).  A and B must each hold
 * bytes_each >= 8192*8192*2 bytes (contents are not used); clk as above
 * (1024 workgroups).  Asynchronous on `stream`.
 *
 * Both return IGC_ERR_INVALID_VALUE for other parameter values or short
 * buffers, IGC_ERR_MISALIGNED for unaligned buffers (4 bytes; A and B 16),
 * IGC_ERR_HIP if the launch fails.
 */
igc_status_t igc_probe_mfma(int mfma, int waves, int iters, int grid, void *sink, int64_t sink_bytes, void *clk,
                            int64_t clk_bytes, igc_stream_t stream);
igc_status_t igc_probe_dma(int bk, int operands, const void *A, const void *B, int64_t bytes_each, void *clk,
                           int64_t clk_bytes, igc_stream_t stream);

/*
 * LDS swizzle of the operand tiles, for inspection and testing on the host.
 * Operand tiles live in LDS as rows of 16-byte chunks; the chunk holding
 * logical chunk `logical_chunk` of row `row` is stored at the returned
 * physical chunk of the same row.  k_contiguous = 1: rows of the K tile
 * (chunks_per_row = BK/8, 8 or 4); 0: rows of BM or BN elements read with the
 * transposing LDS load (chunks_per_row a multiple of 16).  Returns -1 for an
 * unsupported geometry.  These are the maps the kernels use.
 */
int igc_lds_chunk(int k_contiguous, int chunks_per_row, int row, int logical_chunk);

#ifdef __cplusplus
}
#endif

#endif /* IGC_H */
