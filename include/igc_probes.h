/*
 * igc_probes.h -- measurement probes for libigc, built as their own library
 * (libigc_probes.so).  They are not part of the GEMM / convolution ABI: they
 * bound it.  The "B200 TMA Pipeline Designer" page (section "Limitations")
 * says the best pipeline depth must be measured on real shapes and clocks;
 * these give the ceilings the measurements are read against.
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
 * igc_probe_lds: LDS read bandwidth.  `grid` workgroups of 64*waves threads
 * (waves 1..16), each holding a 96 KB LDS buffer (so one workgroup per CU),
 * run `iters` iterations of 8 reads per wave of one kind: kind 0 =
 * ds_read_b128 (16 bytes per lane), 1 = ds_read_b64_tr_b16 (8 bytes), 2 =
 * ds_read_b64 (8 bytes), consecutive lanes on consecutive addresses, i.e.
 * grid*waves*iters*8*64*(16 or 8) bytes.  sink takes one uint32 per thread
 * (grid*64*waves*4 bytes), clk as above.  Asynchronous on `stream`.
 *
 * All three return IGC_ERR_INVALID_VALUE for other parameter values or short
 * buffers, IGC_ERR_MISALIGNED for unaligned buffers (4 bytes; A and B 16),
 * IGC_ERR_HIP if the launch fails.
 */
#ifndef IGC_PROBES_H
#define IGC_PROBES_H

#include "igc.h"

#ifdef __cplusplus
extern "C" {
#endif

igc_status_t igc_probe_mfma(int mfma, int waves, int iters, int grid, void *sink, int64_t sink_bytes, void *clk,
                            int64_t clk_bytes, igc_stream_t stream);
igc_status_t igc_probe_dma(int bk, int operands, const void *A, const void *B, int64_t bytes_each, void *clk,
                           int64_t clk_bytes, igc_stream_t stream);
igc_status_t igc_probe_lds(int kind, int waves, int iters, int grid, void *sink, int64_t sink_bytes, void *clk,
                           int64_t clk_bytes, igc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* IGC_PROBES_H */
