// tile_configs.hpp -- the compiled (BM, BN, BK, PIPE_DEPTH, WAVES, MFMA, HALF,
// LOADERS) configurations; MFMA is the edge of the MFMA block (32: 32x32x16,
// 16: 16x16x32), HALF = 1 gives the ring one operand slot beyond PIPE_DEPTH
// whole stages, and LOADERS waves issue the global->LDS loads (0: every wave).
// Each X(...) line is built as its own object (instances.hip) with every
// operand layout and input type; the build script reads this list.
#pragma once
#define IGC_FOR_EACH_TILE(X)            \
    X(256, 256, 64, 2, 8, 16, 1, 4)     \
    X(256, 256, 32, 4, 8, 16, 0, 4)     \
    X(256, 256, 64, 2, 8, 16, 1, 0)     \
    X(256, 256, 32, 4, 8, 16, 0, 0)     \
    X(256, 256, 64, 2, 8, 32, 1, 4)     \
    X(256, 256, 32, 4, 8, 32, 0, 0)     \
    X(256, 256, 32, 5, 8, 32, 0, 0)     \
    X(256, 256, 64, 2, 4, 32, 1, 0)     \
    X(256, 256, 32, 4, 4, 16, 0, 0)     \
    X(256, 256, 64, 2, 4, 32, 0, 0)     \
    X(256, 256, 64, 1, 4, 32, 0, 0)     \
    X(256, 128, 64, 3, 4, 32, 0, 0)     \
    X(128, 128, 64, 4, 4, 16, 0, 0)     \
    X(128, 128, 64, 4, 4, 32, 0, 0)
