// instances.hpp -- registry of compiled kernel instances (host side).
#pragma once
#include <stdint.h>

#include "igc.h"
#include "tile_configs.hpp"

namespace igc {

struct Instance {
    int bm, bn, bk, d, waves, mfma, half, loaders;
    bool fp16, a_kc, b_kc, conv;
    const void* fn;      // __global__ gemm_kernel<Cfg<...>>
    int64_t lds_bytes;   // static LDS of one workgroup
};

// One table per tile configuration, defined in instances.hip.
#define IGC_DECLARE_TABLE(BM, BN, BK, D, W, MI, H, L) \
    const Instance* instance_table_##BM##x##BN##x##BK##x##D##x##W##x##MI##x##H##x##L(int* count);
IGC_FOR_EACH_TILE(IGC_DECLARE_TABLE)
#undef IGC_DECLARE_TABLE

const Instance* find_instance(const igc_tune_t& t, bool fp16, bool a_kc, bool b_kc, bool conv);
igc_tune_t default_tune(int64_t M, int64_t N, int64_t K, bool conv);
int num_tunes();
igc_tune_t tune_at(int i);

}  // namespace igc
