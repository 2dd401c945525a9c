// tile_configs.hpp -- the compiled (BM, BN, BK, PIPE_DEPTH, WAVES) configurations.
// Each X(...) line is built as its own object (instances.hip) with every
// operand layout and input type; the build script reads this list.
#pragma once
#define IGC_FOR_EACH_TILE(X)  \
    X(256, 256, 32, 5, 8)     \
    X(256, 256, 32, 4, 8)     \
    X(256, 256, 64, 2, 8)     \
    X(256, 256, 32, 5, 4)     \
    X(256, 256, 64, 2, 4)     \
    X(256, 256, 64, 1, 4)     \
    X(256, 128, 64, 3, 4)     \
    X(128, 128, 64, 4, 4)
