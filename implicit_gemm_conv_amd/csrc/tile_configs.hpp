// tile_configs.hpp -- the compiled (BM, BN, BK, PIPE_DEPTH, WAVES, MFMA, HALF,
// LOADERS, SYNC, SCOPE) configurations.  MFMA is the edge of the MFMA block
// (32: 32x32x16, 16: 16x16x32); HALF = 1 gives the ring one operand slot
// beyond PIPE_DEPTH whole stages; LOADERS waves issue the global->LDS loads (0:
// every wave); SYNC 0 meets the workgroup at one barrier per K tile, SYNC 1
// uses per-slot LDS ready/free counters instead.  SCOPE is a bit mask: bit 0
// builds the configuration for every input type, operand layout and operation
// (GEMM, forward convolution, data and filter gradients) with every loop
// variant -- without it only the bf16 and fp16 GEMM with row-major A (both B
// layouts, K a multiple of 8) and the bf16 forward convolution (whole filter
// taps per K tile), which is what the stage-budget, synchronisation and
// small-grid studies time; bit 1 also builds the stream-K kernel; bit 2
// builds those study GEMMs plus the bf16 and fp16 forward convolution with
// every loop variant (for tiles whose rows cannot serve M/N-contiguous
// operands, such as 224-row tiles).  The build script reads this list and
// compiles one object per configuration and operation family.
#pragma once
#define IGC_FOR_EACH_TILE(X)                  \
    X(256, 256, 64, 2, 8, 16, 1, 4, 0, 3)     \
    X(224, 256, 64, 2, 8, 16, 1, 4, 0, 4)     \
    X(128, 64, 64, 2, 4, 16, 0, 0, 0, 4)      \
    X(256, 64, 64, 2, 8, 16, 0, 4, 0, 4)      \
    X(128, 128, 64, 4, 8, 16, 0, 4, 0, 3)     \
    X(256, 256, 32, 4, 8, 16, 0, 4, 0, 3)     \
    X(128, 128, 64, 4, 4, 32, 0, 0, 0, 3)     \
    X(256, 128, 64, 3, 8, 16, 0, 4, 0, 3)     \
    X(256, 256, 32, 2, 8, 32, 0, 4, 0, 0)     \
    X(256, 256, 32, 3, 8, 32, 0, 4, 0, 0)     \
    X(256, 256, 32, 4, 8, 32, 0, 4, 0, 0)     \
    X(256, 256, 32, 5, 8, 32, 0, 4, 0, 0)     \
    X(256, 256, 64, 2, 4, 32, 0, 0, 0, 0)     \
    X(256, 256, 32, 4, 8, 16, 0, 0, 0, 0)     \
    X(256, 256, 32, 4, 8, 16, 0, 4, 1, 2)     \
    X(128, 128, 64, 4, 8, 16, 0, 4, 1, 2)     \
    X(256, 256, 32, 3, 8, 32, 0, 4, 1, 0)     \
    X(256, 256, 32, 4, 8, 32, 0, 4, 1, 0)     \
    X(256, 256, 64, 1, 4, 32, 0, 0, 0, 0)     \
    X(256, 128, 64, 3, 4, 32, 0, 0, 0, 0)
