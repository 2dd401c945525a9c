// instances.hpp -- registry of compiled kernel instances (host side).
#pragma once
#include <stdint.h>

#include "igc.h"
#include "tile_configs.hpp"

namespace igc {

struct Instance {
    int bm, bn, bk, d, waves, mfma, half, loaders, sync;
    int op;              // OpKind: 0 GEMM, 1 forward conv, 2 data gradient, 3 filter gradient
    bool fp16, a_kc, b_kc;
    bool full;           // every loop variant compiled (else only K % 8 == 0 GEMMs and whole-tap convolutions)
    // kernels by loop variant (PLAIN, UNIFORM_TAP, RAGGED, CONV_GENERIC), nullptr where not built:
    const void* fn[4];     // __global__ gemm_kernel<Cfg<...>, V>: data-parallel grid and split-K
    const void* fn_sk[4];  // __global__ gemm_sk_kernel<Cfg<...>, V>: stream-K
    int64_t lds_bytes;   // static LDS of one workgroup
};

// Each compiled object (one configuration, one operation family) registers
// its table when the library is loaded.
void register_instances(const Instance* table, int count);

const Instance* find_instance(const igc_tune_t& t, bool fp16, bool a_kc, bool b_kc, int op);
igc_tune_t default_tune(int64_t M, int64_t N, int64_t K, int op);
int num_tunes();
igc_tune_t tune_at(int i);
int tune_scope(int i);

}  // namespace igc
