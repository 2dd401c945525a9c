// split_reduce.hpp -- host launchers of the split-K reduction and of the
// stream-K flag clearing (split_reduce.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace igc {

// C[m][n] = round(sum_{s<S} ws[s*ws_stride + m*ldws + n]) for m < M, n < N;
// kind 0 = fp32, 1 = bf16, 2 = fp16 output (round to nearest even).
hipError_t launch_split_reduce(const float* ws, int S, int64_t ws_stride, int64_t M, int64_t N, int64_t ldws,
                               void* C, int64_t ldc, int kind, hipStream_t stream);

// Sets flags[0 .. n) to zero, ordered before later work on `stream`.
hipError_t launch_clear_flags(int* flags, int n, hipStream_t stream);

}  // namespace igc
