// probes.hip -- measurement kernels behind the bench's ceilings (not on the
// GEMM path): an MFMA-only stream with the wave tile of the GEMM kernels, and
// the GEMM's global->LDS tile loads without LDS reads or MFMAs.  Both read the
// shader clock in-kernel (s_memtime against the 100 MHz s_memrealtime), since
// the clock under sustained MFMA load sits well below the 2.4 GHz the peak
// assumes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "igc_probes.h"
#include "mainloop.hpp"

namespace igc {

// Operand bits: bf16 values of magnitude in [2^-7, 1) with random sign and
// mantissa (random data, as the GEMM streams; constant operands would let the
// clock float higher than real work allows).
__device__ __forceinline__ i16x8_t probe_bits(uint32_t seed) {
    i16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        seed ^= seed << 13;
        seed ^= seed >> 17;
        seed ^= seed << 5;
        const uint32_t exp = 120u + (seed >> 29);  // 120..127 -> [2^-7, 1)
        v[e] = (short)(((seed & 1u) << 15) | ((exp > 126u ? 126u : exp) << 7) | ((seed >> 8) & 0x7fu));
    }
    return v;
}

template <int MI, int NW>
__global__ __launch_bounds__(64 * NW) void mfma_probe_kernel(float* sink, uint32_t* clk, int iters) {
    using Acc = typename std::conditional<MI == 32, f32x16_t, f32x4_t>::type;
    constexpr int WTM = 128, WTN = NW == 8 ? 64 : 128;  // the GEMM kernels' wave tiles
    constexpr int FM = WTM / MI, FN = WTN / MI;
    const uint32_t gid = blockIdx.x * (64 * NW) + threadIdx.x;
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    i16x8_t a[2][FM], b[2][FN];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < FM; ++i) a[s][i] = probe_bits(gid * 7919u + 131u * (s * 16 + i) + 1u);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[s][j] = probe_bits(gid * 104729u + 257u * (s * 16 + j) + 3u);
    }
    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma<false>(b[s][j], a[s][i], acc[i][j]);
    }
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < (int)(sizeof(Acc) / 4); ++r) x += acc[i][j][r];
    sink[gid] = x;
    __syncthreads();
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = (uint32_t)(c1 - c0);
        clk[2 * blockIdx.x + 1] = (uint32_t)(r1 - r0);
    }
}

// The 8192^3 GEMM's tile loads (A and B row-major bf16, 256 x 256 tiles in the
// GEMM's XCD order, 8 waves), D-slot ring paced by vmcnt with a workgroup
// barrier per K tile; OPS: 1 = A only, 2 = B only, 3 = both.
constexpr int kProbeMN = 8192, kProbeK = 8192;

template <int BK, int D, int OPS>
__global__ __launch_bounds__(512) void dma_probe_kernel(const char* A, const char* B, uint32_t* clk) {
    constexpr int NW = 8;
    constexpr int ABYTES = 256 * BK * 2, BBYTES = BK * 256 * 2;
    constexpr int AI = ABYTES / 1024 / NW, BI = BBYTES / 1024 / NW;
    constexpr int LPT = ((OPS & 1) ? AI : 0) + ((OPS & 2) ? BI : 0);
    constexpr int STAGE = ((OPS & 1) ? ABYTES : 0) + ((OPS & 2) ? BBYTES : 0);
    static_assert(STAGE * D <= 163840 && (D - 1) * LPT < 64, "probe ring");
    __shared__ __attribute__((aligned(1024))) char lds[STAGE * D];
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int tm, tn;
    tile_coords(blockIdx.x, kProbeMN / 256, kProbeMN / 256, 8, tm, tn);
    constexpr int ACPR = BK / 8, ARPI = 64 / ACPR;  // A: 256 rows of BK elements
    constexpr int BCPR = 32, BRPI = 2;              // B: BK rows of 256 elements
    uint32_t aoff[AI], boff[BI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int row = (j * NW + wave) * ARPI + lane / ACPR;
        aoff[j] = (uint32_t)((tm * 256 + row) * kProbeK * 2 + (lane % ACPR) * 16);
    }
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int row = (j * NW + wave) * BRPI + lane / BCPR;
        boff[j] = (uint32_t)(row * kProbeMN * 2 + (tn * 256 + (lane % BCPR) * 8) * 2);
    }
    auto issue = [&](int t, int slot) __attribute__((always_inline)) {
        IGC_LDS char* st = (IGC_LDS char*)lds + slot * STAGE;
        if constexpr (OPS & 1) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(A + (size_t)t * BK * 2);
#pragma unroll
            for (int j = 0; j < AI; ++j) dma16(rs, st + (j * NW + wave) * 1024, aoff[j]);
            st += ABYTES;
        }
        if constexpr (OPS & 2) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(B + (size_t)t * BK * kProbeMN * 2);
#pragma unroll
            for (int j = 0; j < BI; ++j) dma16(rs, st + (j * NW + wave) * 1024, boff[j]);
        }
    };
    constexpr int KT = kProbeK / BK;
#pragma unroll
    for (int s = 0; s < D - 1; ++s) issue(s, s);
    for (int t0 = 0; t0 < KT; t0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int t = t0 + u;
            if (t + D - 1 < KT) issue(t + D - 1, (u + D - 1) % D);
            if (t + D - 1 < KT)
                wait_vmcnt<(D - 1) * LPT>();  // tile t landed: loads complete in order
            else
                wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
        }
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = (uint32_t)(c1 - c0);
        clk[2 * blockIdx.x + 1] = (uint32_t)(r1 - r0);
    }
}

// LDS read bandwidth: every wave streams reads of one kind over a 96 KB LDS
// buffer (more than half the CU's LDS, so one workgroup per CU) with
// consecutive lanes on consecutive addresses; KIND 0 = ds_read_b128 (the
// GEMM's K-contiguous fragments), 1 = ds_read_b64_tr_b16 (its M/N-contiguous
// fragments), 2 = ds_read_b64.
constexpr int kLdsProbeBytes = 96 * 1024;

template <int KIND>
__global__ __launch_bounds__(1024) void lds_probe_kernel(uint32_t* sink, uint32_t* clk, int iters) {
    __shared__ __attribute__((aligned(1024))) char lds[kLdsProbeBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int i = threadIdx.x * 4; i < kLdsProbeBytes; i += blockDim.x * 4) *(uint32_t*)(lds + i) = i * 2654435761u;
    __syncthreads();
    constexpr int BPL = KIND == 0 ? 16 : 8;  // bytes per lane
    constexpr int PER = 64 * BPL;            // bytes per wave instruction
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    uint32_t x = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // (it * 8 + j) * nw + wave instruction slots, wrapped inside the buffer
            const uint32_t off = ((uint32_t)((it * 8 + j) * nw + wave) * PER) % kLdsProbeBytes + lane * BPL;
            if constexpr (KIND == 0) {
                const i16x8_t v = *(IGC_LDS i16x8_t*)((IGC_LDS char*)lds + off);
                x ^= (uint32_t)v[0] ^ ((uint32_t)v[7] << 16);
            } else if constexpr (KIND == 1) {
                const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((IGC_LDS i16x4_t*)((IGC_LDS char*)lds + off));
                x ^= (uint32_t)v[0] ^ ((uint32_t)v[3] << 16);
            } else {
                const i16x4_t v = *(IGC_LDS i16x4_t*)((IGC_LDS char*)lds + off);
                x ^= (uint32_t)v[0] ^ ((uint32_t)v[3] << 16);
            }
        }
    }
    sink[blockIdx.x * blockDim.x + threadIdx.x] = x;
    __syncthreads();
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = (uint32_t)(c1 - c0);
        clk[2 * blockIdx.x + 1] = (uint32_t)(r1 - r0);
    }
}

}  // namespace igc

using namespace igc;

extern "C" {

igc_status_t igc_probe_mfma(int mfma, int waves, int iters, int grid, void* sink, int64_t sink_bytes, void* clk,
                            int64_t clk_bytes, igc_stream_t stream) {
    if ((mfma != 16 && mfma != 32) || (waves != 4 && waves != 8) || iters < 1 || grid < 1 || !sink || !clk)
        return IGC_ERR_INVALID_VALUE;
    if (sink_bytes < (int64_t)grid * 64 * waves * 4 || clk_bytes < (int64_t)grid * 8) return IGC_ERR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(sink) & 3) || (reinterpret_cast<uintptr_t>(clk) & 3)) return IGC_ERR_MISALIGNED;
    const void* fn = mfma == 16 ? (waves == 8 ? (const void*)&mfma_probe_kernel<16, 8> : (const void*)&mfma_probe_kernel<16, 4>)
                                : (waves == 8 ? (const void*)&mfma_probe_kernel<32, 8> : (const void*)&mfma_probe_kernel<32, 4>);
    float* s = (float*)sink;
    uint32_t* c = (uint32_t*)clk;
    void* args[] = {&s, &c, &iters};
    (void)hipGetLastError();
    if (hipLaunchKernel(fn, dim3(grid), dim3(64 * waves), args, 0, (hipStream_t)stream) != hipSuccess)
        return IGC_ERR_HIP;
    return IGC_OK;
}

igc_status_t igc_probe_dma(int bk, int operands, const void* A, const void* B, int64_t bytes_each, void* clk,
                           int64_t clk_bytes, igc_stream_t stream) {
    constexpr int grid = (kProbeMN / 256) * (kProbeMN / 256);
    if ((bk != 16 && bk != 32 && bk != 64) || operands < 1 || operands > 3 || !A || !B || !clk)
        return IGC_ERR_INVALID_VALUE;
    if (bytes_each < (int64_t)kProbeMN * kProbeK * 2 || clk_bytes < (int64_t)grid * 8) return IGC_ERR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(B) & 15) ||
        (reinterpret_cast<uintptr_t>(clk) & 3))
        return IGC_ERR_MISALIGNED;
    const void* table[3][3] = {
        {(const void*)&dma_probe_kernel<16, 4, 1>, (const void*)&dma_probe_kernel<16, 4, 2>,
         (const void*)&dma_probe_kernel<16, 4, 3>},
        {(const void*)&dma_probe_kernel<32, 4, 1>, (const void*)&dma_probe_kernel<32, 4, 2>,
         (const void*)&dma_probe_kernel<32, 4, 3>},
        {(const void*)&dma_probe_kernel<64, 2, 1>, (const void*)&dma_probe_kernel<64, 2, 2>,
         (const void*)&dma_probe_kernel<64, 2, 3>}};
    const void* fn = table[bk == 16 ? 0 : (bk == 32 ? 1 : 2)][operands - 1];
    const char* a = (const char*)A;
    const char* b = (const char*)B;
    uint32_t* c = (uint32_t*)clk;
    void* args[] = {&a, &b, &c};
    (void)hipGetLastError();
    if (hipLaunchKernel(fn, dim3(grid), dim3(512), args, 0, (hipStream_t)stream) != hipSuccess) return IGC_ERR_HIP;
    return IGC_OK;
}

igc_status_t igc_probe_lds(int kind, int waves, int iters, int grid, void* sink, int64_t sink_bytes, void* clk,
                           int64_t clk_bytes, igc_stream_t stream) {
    if (kind < 0 || kind > 2 || waves < 1 || waves > 16 || iters < 1 || grid < 1 || !sink || !clk)
        return IGC_ERR_INVALID_VALUE;
    if (sink_bytes < (int64_t)grid * 64 * waves * 4 || clk_bytes < (int64_t)grid * 8) return IGC_ERR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(sink) & 3) || (reinterpret_cast<uintptr_t>(clk) & 3)) return IGC_ERR_MISALIGNED;
    const void* fn = kind == 0 ? (const void*)&lds_probe_kernel<0>
                               : (kind == 1 ? (const void*)&lds_probe_kernel<1> : (const void*)&lds_probe_kernel<2>);
    uint32_t* s = (uint32_t*)sink;
    uint32_t* c = (uint32_t*)clk;
    void* args[] = {&s, &c, &iters};
    (void)hipGetLastError();
    if (hipLaunchKernel(fn, dim3(grid), dim3(64 * waves), args, 0, (hipStream_t)stream) != hipSuccess)
        return IGC_ERR_HIP;
    return IGC_OK;
}

}  // extern "C"
