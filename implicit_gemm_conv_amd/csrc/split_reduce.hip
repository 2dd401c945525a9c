// split_reduce.hip -- second pass of split-K: C = sum over splits of the fp32
// partial tiles, added in split order 0, 1, ..., S-1 (fixed, so results are
// bit-reproducible), then rounded once to the output type.  Also the small
// kernel that clears the stream-K flags before a stream-K launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "split_reduce.hpp"

namespace igc {

typedef __attribute__((ext_vector_type(4))) float f32x4r_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4r_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4r_t;

// One thread per 4 consecutive outputs of a row.  The partials are read four
// splits at a time (independent 16-byte loads) and added in split order, so the
// sum is the same as one add per split in sequence.  VEC: C's rows and base are
// aligned for one 16-byte (fp32) or 8-byte (16-bit) store per thread, done when
// all 4 outputs lie inside the row.
template <bool VEC>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ ws, int S, int64_t ws_stride,
                                                           int64_t M, int64_t N, int64_t ldws, void* C,
                                                           int64_t ldc, int kind) {
    const int64_t n4 = (N + 3) / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * n4) return;
    int64_t m;
    if (M * n4 <= 0xffffffffLL)
        m = (uint32_t)idx / (uint32_t)n4;  // 32-bit division when the index fits
    else
        m = idx / n4;
    const int64_t n = (idx - m * n4) * 4;
    // ldws is a multiple of 4 and >= N rounded up to 4: the 16-byte read stays in the row
    const float* src = ws + m * ldws + n;
    f32x4r_t acc = *(const f32x4r_t*)src;
    int s = 1;
    for (; s + 3 < S; s += 4) {
        const f32x4r_t a1 = *(const f32x4r_t*)(src + s * ws_stride);
        const f32x4r_t a2 = *(const f32x4r_t*)(src + (s + 1) * ws_stride);
        const f32x4r_t a3 = *(const f32x4r_t*)(src + (s + 2) * ws_stride);
        const f32x4r_t a4 = *(const f32x4r_t*)(src + (s + 3) * ws_stride);
        acc += a1;
        acc += a2;
        acc += a3;
        acc += a4;
    }
    for (; s < S; ++s) acc += *(const f32x4r_t*)(src + s * ws_stride);
    const int64_t off = m * ldc + n;
    if (VEC && n + 4 <= N) {
        if (kind == 0) {
            *(f32x4r_t*)((float*)C + off) = acc;
        } else if (kind == 1) {
            bf16x4r_t v;
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[e];
            *(bf16x4r_t*)((__bf16*)C + off) = v;
        } else {
            f16x4r_t v;
            for (int e = 0; e < 4; ++e) v[e] = (_Float16)acc[e];
            *(f16x4r_t*)((_Float16*)C + off) = v;
        }
        return;
    }
    for (int e = 0; e < 4; ++e) {
        if (n + e >= N) break;
        if (kind == 0)
            ((float*)C)[off + e] = acc[e];
        else if (kind == 1)
            ((__bf16*)C)[off + e] = (__bf16)acc[e];
        else
            ((_Float16*)C)[off + e] = (_Float16)acc[e];
    }
}

hipError_t launch_split_reduce(const float* ws, int S, int64_t ws_stride, int64_t M, int64_t N, int64_t ldws,
                               void* C, int64_t ldc, int kind, hipStream_t stream) {
    const int64_t work = M * ((N + 3) / 4);
    if (work <= 0) return hipSuccess;
    const int64_t blocks = (work + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    // a thread's 4 outputs start at element m*ldc + 4j: aligned for one store when ldc is a multiple
    // of 4 and the base is aligned to the store's width (16 bytes for fp32, 8 for 16-bit outputs)
    const uintptr_t width = kind == 0 ? 16 : 8;
    const bool vec = ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % width == 0;
    if (vec)
        hipLaunchKernelGGL(split_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, ws, S, ws_stride,
                           M, N, ldws, C, ldc, kind);
    else
        hipLaunchKernelGGL(split_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, ws, S,
                           ws_stride, M, N, ldws, C, ldc, kind);
    return hipGetLastError();
}

// Zeroes n stream-K flags.  System-coherent stores (SC0 | SC1) write through
// to memory, so the next kernel's flag polls on any XCD see the zero.
__global__ __launch_bounds__(256) void sk_clear_flags_kernel(int* flags, int n) {
    const int i = (int)(blockIdx.x * 256 + threadIdx.x);
    if (i < n)
        __builtin_amdgcn_raw_buffer_store_b32(
            0, __builtin_amdgcn_make_buffer_rsrc(flags, (short)0, 0x7fffffff, 0x00020000), i * 4, 0, 1 | 16);
}

hipError_t launch_clear_flags(int* flags, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(sk_clear_flags_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, flags, n);
    return hipGetLastError();
}

}  // namespace igc
