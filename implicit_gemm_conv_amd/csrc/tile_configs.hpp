// tile_configs.hpp -- the compiled (BM, BN, BK, PIPE_DEPTH) configurations.
// Each X(...) line is built as its own object (instances.hip) with every
// operand layout and input type; the build script reads this list.
#pragma once
#define IGC_FOR_EACH_TILE(X) \
    X(256, 256, 64, 2)       \
    X(256, 256, 32, 4)       \
    X(256, 256, 64, 1)       \
    X(256, 128, 64, 3)       \
    X(128, 128, 64, 4)
