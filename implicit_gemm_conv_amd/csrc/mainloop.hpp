// mainloop.hpp -- the software-pipelined bf16/fp16 MFMA mainloop for gfx950.
//
// One workgroup of 4 or 8 wave64s computes a BM x BN tile of C = A * B (or of
// the implicit-GEMM view of an NHWC convolution).  Waves form a 2 x (NW/2)
// grid; each owns a sub-tile held as MI x MI MFMA blocks (MI = 32 or 16) of
// fp32 accumulators in registers for the whole K loop.
//
// Subsystems (the "B200 TMA Pipeline Designer" page, Executable steps 2-7,
// re-done for CDNA4):
//  1. Stage ring: PIPE_DEPTH LDS stages, each its own __shared__ array so that
//     every slot index is a compile-time constant after unrolling the K loop by
//     PIPE_DEPTH; the compiler then proves the direct-to-LDS writes into one
//     slot do not alias the ds_reads of another and emits no conservative
//     vmcnt(0).  Operand tiles move global -> LDS with buffer_load_dwordx4 ...
//     lds (16 B per lane, written at M0 + 16*lane), one 1 KB wave instruction
//     at a time; out-of-range chunks get an out-of-bounds buffer offset and
//     land as zeros (the tile boundary policy).  Schedule: ring.hpp.
//  2. Swizzle: the direct-to-LDS destination is fixed, so the XOR swizzle is
//     applied on the global side (which 16-byte chunk each lane fetches) and
//     undone by the fragment reader with the same map.  K-contiguous tiles
//     (rows of BK elements) XOR the chunk index with (row>>1)&7 for BK = 64,
//     or (-(row>>2))&3 for BK = 32; M/N-contiguous tiles (rows of BM or BN
//     elements, read with the transposing ds_read_b64_tr_b16) XOR it with
//     4*(row&3) + 2*((row>>3)&1).  Each map makes every lane phase of a
//     fragment read hit distinct banks for both MFMA shapes.
//  3. MFMA loop: v_mfma_f32_32x32x16 or v_mfma_f32_16x16x32, {bf16,f16}; each
//     lane holds 8 consecutive k of one row/column per operand.  B is passed
//     as the first operand so that each lane's 4 consecutive accumulators are
//     4 consecutive output columns (vector stores in the epilogue).  Both
//     shapes run at the same rate per clock, but the 16x16x32 form rewrites
//     its accumulators half as often per flop (K = 32 per instruction), and
//     under sustained load it holds a markedly higher clock on gfx950.
//  4. Boundary: rows/columns past M/N and k past K load as zeros; when K is not
//     a multiple of 8 the lane that loaded a chunk straddling K zeroes its tail
//     in LDS after its own wait and before the barrier.  The epilogue stores
//     only in-range elements (full tiles take an unmasked vector path).
//  5. im2col: for the convolution, each A row (output pixel n,p,q) and K chunk
//     (tap r,s and 8 channels) maps to x[n][p*sh-ph+r*dh][q*sw-pw+s*dw][c..c+7],
//     or to the out-of-bounds offset when the tap falls in the zero padding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fastdiv.hpp"
#include "ring.hpp"

namespace igc {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

#define IGC_LDS __attribute__((address_space(3)))

template <int I>
struct IntC {
    static constexpr int value = I;
    constexpr operator int() const { return I; }
};
// Calls f(IntC<B>{}), ..., f(IntC<E-1>{}): the index is a compile-time constant in the body.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}

constexpr uint32_t kOob = 0x80000000u;          // buffer offset that is always out of range
constexpr int kNumRecords = 0x7fffffff;         // range of every buffer resource
constexpr int kRsrcFlags = 0x00020000;          // gfx9 raw buffer: 32-bit dword format

enum OutKind : int { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

// What the mainloop computes.  Every operation is one GEMM C = A * B whose
// operands are read in place; the convolutions differ only in how a tile's
// rows and K indices map to addresses (the implicit-GEMM views):
//   OP_GEMM : A (M x K) and B (K x N) dense, either layout.
//   OP_FPROP: forward convolution.  Rows m = output pixels (n, p, q), K index
//             = (filter tap, input channel); A gathers x (NHWC, channel
//             contiguous), B = w as an N x K column-major matrix (KRSC).
//   OP_DGRAD: data gradient.  Rows m = input pixels (n, h, w), K index =
//             (filter tap, output channel); A gathers dy (NPQK) at the output
//             pixel whose forward window puts that tap on (h, w), B row k*R*S
//             + tap of w (KRSC) holds that tap's C input channels contiguously.
//   OP_WGRAD: filter gradient.  Rows m = output channels, columns = (tap,
//             input channel), K index = output pixels (n, p, q); A = dy read
//             column-major (NPQK), B gathers x at each pixel's tap position.
enum OpKind : int { OP_GEMM = 0, OP_FPROP = 1, OP_DGRAD = 2, OP_WGRAD = 3 };

struct Params {
    const void* A;   // GEMM A; conv: x (FPROP), dy (DGRAD, WGRAD)
    const void* B;   // GEMM B; conv: w (FPROP, DGRAD), x (WGRAD)
    void* C;         // row-major M x N (FPROP: y NPQK; DGRAD: dx NHWC; WGRAD: dw KRSC)
    int64_t M, N, K; // GEMM view
    int64_t lda, ldb, ldc;
    int tiles_m, tiles_n;
    int out_kind;
    int group_m;     // tiles of M walked together inside one XCD's range (L2 reuse)
    // split-K: k_splits workgroups share each output tile, split s covering
    // K in [s*k_per_split, min(K, (s+1)*k_per_split)); each writes its fp32
    // partial tile to ws + s*ws_stride (row pitch ldws) instead of C.
    int k_splits;
    int64_t k_per_split;
    float* ws;
    int64_t ldws, ws_stride;
    int k_ragged8;   // K % 8 != 0: chunk straddling K must be zeroed
    int vec_ok;      // output rows allow 8/16-byte vector stores
    // convolution geometry: input N x H x W x Cin, filter R x S, output P x Q x Kc
    int H, W, Cin, Kc, R, S, P, Q, sh, sw, ph, pw, dh, dw;
    // The gathered operand of FPROP and DGRAD (A, channel contiguous): the
    // image it reads (gH x gW pixels of gC channels), the pixel grid of the
    // GEMM rows (rP x rQ), where row pixel (a, b) puts filter tap (0, 0)
    // (a*rsh + roh, b*rsw + row) and how far one filter row / column moves in
    // the image (tdh, tdw).  FPROP: x, rows over P x Q, (a*sh - ph, b*sw - pw),
    // steps (dh, dw).  DGRAD: dy, rows over H x W, (a + ph, b + pw), steps
    // (-dh, -dw), and a landing position is an image row/column only when it
    // is a multiple of the stride (gsh, gsw; 1 for FPROP).
    int gH, gW, gC, rP, rQ, rsh, rsw, roh, row, tdh, tdw, gsh, gsw;
    uint32_t gsh_magic, gsw_magic;
    // stream-K (sk_grid > 0 persistent workgroups).  Workgroup g first runs
    // whole tiles g, g+G, ... below sk_dp_tiles (data-parallel rounds), then
    // the K ranges of the remaining tiles, in units of the ring period
    // (sk_units per tile), cut into sk_grid equal runs: a workgroup whose run
    // ends inside a tile publishes an fp32 partial tile in sk_ws (one BM x BN
    // slot per workgroup) and raises its flag sk_flags[g] to 1; the workgroup
    // that computes the tile's last K unit adds the partials of the lower
    // workgroups in descending order and stores the tile.  The flags are
    // cleared by a kernel launched just before on the same stream.
    int sk_grid;
    int64_t sk_units;
    int64_t sk_dp_tiles;
    float* sk_ws;
    int* sk_flags;
    int sk_spin_limit;  // polls of a flag before the owner gives up
    int sk_drop;        // test hook: the workgroup whose flag is never raised (-1: none)
    int* err_word;      // set to 1 when a bounded wait gives up (the tile is then written as NaN)
    int conv_uniform;  // gC % BK == 0: every K tile lies within one filter tap
    int conv_masks;    // unit stride (DGRAD), R <= 16 and S <= 16: tap validity from per-row bit masks
    int tpt;           // K tiles per filter tap (gC / BK) when conv_uniform
    uint32_t cin_magic, s_magic, tpt_magic;  // fastdiv multipliers for gC, S and tpt
    uint32_t q_magic, pq_magic;              // WGRAD pixel decode: Q and P*Q
};

// Loop variants, chosen per call and compiled as separate loops so that none
// carries a branch between its MFMAs: GEMM with K % 8 == 0 or convolution
// whose channel tiles straddle filter taps (PLAIN), K % 8 != 0 (RAGGED),
// convolution with whole filter taps per K tile (UNIFORM_TAP), and convolution
// with a filter wider or taller than 16 taps or a strided data gradient
// (CONV_GENERIC; the others keep a per-row bit mask of the filter rows and
// columns that fall inside the image).  The filter gradient has one form.
enum LoopVariant : int { PLAIN = 0, UNIFORM_TAP = 1, RAGGED = 2, CONV_GENERIC = 3 };

// XOR swizzle of the 16-byte chunk index within a K-contiguous LDS row of CPR
// chunks.  On gfx950 the LDS serves a 128-bit read 16 lanes at a time over its
// 64 banks (256 bytes); the 16 lanes of a phase are four lane quads of equal
// quad parity, e.g. lanes {0-3, 12-15, 20-23, 24-27} (measured with the bank
// conflict counter).  A 32x32x16 fragment read puts lane l on row l%32 at
// logical chunk 2kk + l/32, a 16x16x32 one on row l%16 at chunk 4kk + l/16;
// both must give each phase 16 distinct (row, chunk) bank groups.  The maps
// depend on row % 16 only, so every 16-row fragment sees the same pattern.
template <int CPR>
IGC_HD inline int swz_k(int row) {
    static_assert(CPR == 8 || CPR == 4, "K tile of 64 or 32 elements");
    if constexpr (CPR == 8) {
        return (row >> 1) & 7;  // 128-byte rows
    } else {
        return (-(row >> 2)) & 3;  // 64-byte rows, four per 256 bytes
    }
}
// XOR swizzle of the 16-byte chunk index within an M/N-contiguous LDS row of
// CPR chunks (8, or a multiple of 16).  ds_read_b64_tr_b16 serves 32 lanes per
// phase; a 32x32x16 fragment read covers 4 k-rows x 4 chunks per phase, a
// 16x16x32 one 8 k-rows (r and r+8, r = 0..3) x 2 chunks.  Rows of 256 bytes
// or more all start on bank 0, so the 8 k-rows of a phase need 8 distinct
// chunk pairs (and quads), which 4*(r&3) + 2*bit3 gives.  Rows of 128 bytes
// alternate between the two halves of the 64 banks, so only rows of equal
// parity compete: 4*bit1 + 2*bit3 separates rows 0, 2, 8 and 10 (and 1, 3, 9,
// 11) into distinct pairs and rows 0 and 2 into distinct quads.  Neither map
// uses a row bit other than 0, 1 and 3, and both stay inside the row.
template <int CPR>
IGC_HD inline int swz_mn(int row) {
    static_assert(CPR == 8 || CPR % 16 == 0, "M/N-contiguous rows of 64 elements or a multiple of 128");
    if constexpr (CPR == 8)
        return 4 * ((row >> 1) & 1) + 2 * ((row >> 3) & 1);
    else
        return 4 * (row & 3) + 2 * ((row >> 3) & 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kNumRecords, kRsrcFlags);
}

// A buffer resource whose base is pinned to scalar registers at its point of
// use.  The base of every operand tile is uniform, but when the compiler
// computes it in vector registers (a 64-bit product, or a value that register
// pressure moved there) it must wrap each load in a waterfall loop; taking the
// two address words through readfirstlane keeps the resource scalar.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void* base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, IGC_LDS void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4]<<14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }  // lgkmcnt(0) only

// MFMA 32x32x16 (16 accumulators per lane) or 16x16x32 (4 per lane), fp32
// accumulate; the accumulator type selects the shape.
template <bool FP16>
__device__ __forceinline__ f32x16_t mfma(i16x8_t a, i16x8_t b, f32x16_t c) {
    if constexpr (FP16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}
template <bool FP16>
__device__ __forceinline__ f32x4_t mfma(i16x8_t a, i16x8_t b, f32x4_t c) {
    if constexpr (FP16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// Operand tile geometry.  ROWS = BM (operand A) or BN (operand B).
//   KC = true : LDS tile is ROWS rows of BK elements (K contiguous).
//   KC = false: LDS tile is BK rows of ROWS elements (M or N contiguous).
// ---------------------------------------------------------------------------
template <int ROWS, int BK, bool KC, int NL>
struct Tile {
    static constexpr int BYTES = ROWS * BK * 2;
    static constexpr int INSTR = BYTES / 1024;        // 1 KB wave instructions per stage
    static constexpr int IPW = INSTR / NL;            // per loading wave
    static constexpr int ROW_ELEMS = KC ? BK : ROWS;  // elements per LDS row
    static constexpr int CPR = ROW_ELEMS / 8;         // 16-byte chunks per LDS row
    static constexpr int RPI = 64 / CPR;              // LDS rows per wave instruction
    static_assert(BYTES % (1024 * NL) == 0, "tile must split into whole wave instructions");
    static_assert(CPR >= 1 && CPR <= 64 && 64 % CPR == 0, "row must be 8..512 elements");
    // LDS row, physical chunk and logical chunk written by `lane` in wave instruction q.
    __device__ static int row_of(int q, int lane) { return q * RPI + lane / CPR; }
    __device__ static int logical_chunk(int q, int lane) {
        const int row = row_of(q, lane);
        if constexpr (KC) {
            return (lane % CPR) ^ swz_k<CPR>(row);
        } else {
            return (lane % CPR) ^ swz_mn<CPR>(row);
        }
    }
};

template <bool FP16_, int BM_, int BN_, int BK_, int D_, int NW_, int MI_, int HALF_, int NL_, int SYNC_, bool A_KC_,
          bool B_KC_, int OPK_>
struct Cfg {
    static constexpr bool FP16 = FP16_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, D = D_;
    // The ring holds U = 2*D + HALF operand slots: A(t) is unit 2t and B(t)
    // unit 2t+1 of a sequence whose unit s lives in slot s % U (ring.hpp).
    static constexpr int HALF = HALF_;
    static constexpr int U = 2 * D_ + HALF_;
    // MFMA block edge: 32 (32x32x16) or 16 (16x16x32)
    static constexpr int MI = MI_;
    static_assert(MI == 32 || MI == 16, "32x32x16 or 16x16x32 MFMA");
    static constexpr int KS = MI == 32 ? 16 : 32;     // K depth of one MFMA (one k-step)
    static constexpr int NH = 64 / MI;                // lane groups per fragment: 16-byte chunks per k-step
    using Acc = typename std::conditional<MI == 32, f32x16_t, f32x4_t>::type;
    // NW wave64s in a 2 x (NW/2) grid.  With 8 waves two share each SIMD, so
    // while one waits to issue a global->LDS load the other keeps the SIMD's
    // matrix core busy.
    static constexpr int NW = NW_, NT = 64 * NW_;
    static constexpr int WM = 2, WN = NW_ / 2;
    // NL loading waves (0: all) issue every global->LDS load of a tile (waves
    // 0 .. NL-1, one per SIMD when NL = 4 of 8); the others only read LDS and
    // run MFMAs, so a SIMD always has a wave whose MFMA issue never waits
    // behind the load path.
    static constexpr int NL = NL_ == 0 ? NW_ : NL_;
    static_assert(NL >= 1 && NL <= NW_ && NW_ % NL == 0, "loading waves divide the workgroup");
    // SPREAD: the two operand slots freed at the barrier before tile t are
    // refilled by loads interleaved through tile t's k-steps, instead of one
    // burst after the barrier.
    static constexpr bool SPREAD = Ring::spread(U);
    static constexpr bool A_KC = A_KC_, B_KC = B_KC_;
    static constexpr int OPK = OPK_;
    static constexpr bool FPROP = OPK == OP_FPROP, DGRAD = OPK == OP_DGRAD, WGRAD = OPK == OP_WGRAD;
    // the operand gathered through an im2col map with per-row tap masks (A of FPROP and DGRAD)
    static constexpr bool GATHER_A = FPROP || DGRAD;
    static_assert(OPK == OP_GEMM || (FPROP && A_KC && B_KC) || (DGRAD && A_KC && !B_KC) || (WGRAD && !A_KC && !B_KC),
                  "operand layouts of the convolution views");
    // SYNC 0: one workgroup barrier per K tile is both "ready" and "free".
    // SYNC 1: per-slot LDS counters -- loading waves count a slot ready once
    // their loads into it have landed, every wave counts it free once its
    // reads of it are done, and waves wait only on the counter they need.
    static constexpr int SYNC = SYNC_;
    static_assert(SYNC == 0 || SYNC == 1, "barrier ring or counter ring");
    static_assert(SYNC == 0 || (U >= 6 && U % 2 == 0), "the counter ring runs whole stages refilled during compute");
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave sub-tile is whole MFMA blocks");
    static constexpr int FM = WTM / MI, FN = WTN / MI;
    static constexpr int KK = BK / KS;                // MFMA k-steps per K tile
    static_assert(KK >= 1 && BK % KS == 0, "K tile is whole k-steps");
    using TA = Tile<BM, BK, A_KC, NL>;
    using TB = Tile<BN, BK, B_KC, NL>;
    // Slot s holds A units when s is even and U is even, B units when s is
    // odd and U is even; with U odd both operands rotate through every slot.
    static constexpr int SLOT_A = TA::BYTES, SLOT_B = TB::BYTES;
    static constexpr int SLOT_MAX = SLOT_A > SLOT_B ? SLOT_A : SLOT_B;
    template <int S>
    static constexpr int slot_bytes() { return U % 2 ? SLOT_MAX : (S % 2 ? SLOT_B : SLOT_A); }
    // the ring, plus the per-stage ready and free counters of SYNC 1
    static constexpr int LDS_BYTES = (U % 2 ? U * SLOT_MAX : D * (SLOT_A + SLOT_B)) + (SYNC_ ? 8 * D_ : 0);
    static constexpr int LPT = TA::IPW + TB::IPW;     // loads per K tile per wave
    // the slot pattern repeats every P tiles; the K loop is unrolled by P
    static constexpr int P = Ring::period(U);
    static_assert(HALF == 0 || HALF == 1, "at most one extra operand slot");
    static_assert(HALF == 0 || D >= 2, "an odd ring needs at least five operand slots");
    // fragments alternate between two register sets by k-step, so one period
    // of the unrolled loop must hold an even number of k-steps
    static_assert((P * KK) % 2 == 0, "fragment double-buffer parity needs an even number of k-steps per period");
    static_assert(D >= 1 && D <= 8, "pipe depth");
    static_assert(LDS_BYTES <= 163840, "stage ring exceeds the 160 KB of LDS per CU");
    static_assert(!SPREAD || Ring::wait_units(U) * (TA::IPW > TB::IPW ? TA::IPW : TB::IPW) < 64,
                  "vmcnt cannot express that many loads in flight");
    static_assert(SPREAD || HALF == 0, "odd rings are refilled during compute");
};

// Per-lane DMA state of one operand: offsets of the chunks this lane fetches
// for each of its wave instructions, relative to a per-tile buffer base.
template <int IPW>
struct DmaState {
    uint32_t voff[IPW];
};

// ---------------------------------------------------------------------------
// The kernel body.
// ---------------------------------------------------------------------------
template <class C, int V, bool LOADER = true>
struct Mainloop {
    static constexpr bool kRagged = V == RAGGED, kUniformTap = V == UNIFORM_TAP;
    static constexpr bool kConvMasks = C::GATHER_A && V != CONV_GENERIC;
    static constexpr bool kConvGeneric = C::GATHER_A && V == CONV_GENERIC;
    // LOADER: this wave issues global->LDS loads (waves 0 .. NL-1)
    using TA = typename C::TA;
    using TB = typename C::TB;
    static constexpr int BM = C::BM, BN = C::BN, BK = C::BK, D = C::D, KK = C::KK;
    static constexpr int FM = C::FM, FN = C::FN, MI = C::MI, KS = C::KS, NH = C::NH;
    using Acc = typename C::Acc;

    // ---- per-workgroup setup -------------------------------------------------
    const Params p;  // a copy: kernel arguments stay in scalar registers
    int lane, wave, wm, wn;
    int64_t m0, n0;  // tile origin
    int64_t kbase, kend;  // this workgroup's K range
    int KT;          // number of K tiles
    int KTp;         // KT rounded up to a multiple of the ring period (padding tiles load zeros)
    DmaState<TA::IPW> da;
    DmaState<TB::IPW> db;
    // im2col (A of FPROP and DGRAD): per A instruction, the row pixel's gather state.
    // masked form: byte offset of the row's pixel at filter tap (0, 0) (may be
    // negative at the padding) and its tap mask (bit r: filter row r lands in
    // the image; bit 16+s: filter column s does; 0 for rows past M)
    int conv_base[kConvMasks ? TA::IPW : 1];
    uint32_t conv_mask[kConvMasks ? TA::IPW : 1];
    // generic form: image base, top-left landing row and column of the window
    int conv_pix[kConvGeneric ? TA::IPW : 1];
    int conv_h0[kConvGeneric ? TA::IPW : 1];
    int conv_w0[kConvGeneric ? TA::IPW : 1];
    // DGRAD B, taps straddling K tiles: the byte offset of the lane's columns (or kOob)
    uint32_t dg_col[C::DGRAD && !kUniformTap ? TB::IPW : 1];
    // WGRAD B: per B instruction, the lane's column as a tap offset in the
    // window (filter row r*dh, column s*dw; r*dh is huge for columns past N)
    // and its channel byte offset
    int wg_rd[C::WGRAD ? TB::IPW : 1];
    int wg_sd[C::WGRAD ? TB::IPW : 1];
    int wg_c2[C::WGRAD ? TB::IPW : 1];
    // the swizzled K chunk this lane fetches (same for all its loads of an operand)
    int ca_lane = 0, cb_lane = 0;
    // fragment read offsets (bytes within a stage's operand region)
    uint32_t fa_off[C::A_KC ? KK : FM];
    uint32_t fb_off[C::B_KC ? KK : FN];

    __device__ __forceinline__ Mainloop(const Params p_, int64_t m0_, int64_t n0_, int64_t kbase_, int64_t kend_)
        : p(p_), m0(m0_), n0(n0_), kbase(kbase_), kend(kend_) {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        wm = wave / C::WN;
        wn = wave % C::WN;
        KT = (int)((kend - kbase + BK - 1) / BK);
        KTp = (KT + C::P - 1) / C::P * C::P;
        setup_dma();
        setup_frag_offsets();
        if constexpr (C::A_KC) ca_lane = TA::logical_chunk(wave, lane);
        // every load of a lane sits 16*k rows below its first, and the K
        // swizzle depends on row % 16 only: one logical chunk per lane
        static_assert(!C::A_KC || (C::NL * TA::RPI) % 16 == 0, "a lane's A chunk must not change between its loads");
        if constexpr (C::B_KC) cb_lane = TB::logical_chunk(wave, lane);
    }

    __device__ __forceinline__ void setup_dma() {
        // Operand A
#pragma unroll
        for (int j = 0; j < TA::IPW; ++j) {
            const int q = j * C::NL + wave;
            const int row = TA::row_of(q, lane);
            const int c = TA::logical_chunk(q, lane);
            if constexpr (C::GATHER_A) {
                // row m = pixel (n, a, b) of the rP x rQ grid; filter tap (0, 0)
                // lands on (h0, w0) of the gathered gH x gW image
                const int64_t m = m0 + row;
                const int PQ = p.rP * p.rQ;
                const int mm = (int)(m < p.M ? m : 0);
                const int n = mm / PQ, pq = mm - n * PQ;
                const int pa = pq / p.rQ, pb = pq - pa * p.rQ;
                const int h0 = pa * p.rsh + p.roh, w0 = pb * p.rsw + p.row;
                if constexpr (kConvMasks) {
                    uint32_t mask = 0;
                    for (int r = 0; r < p.R; ++r)
                        if ((unsigned)(h0 + r * p.tdh) < (unsigned)p.gH) mask |= 1u << r;
                    for (int s = 0; s < p.S; ++s)
                        if ((unsigned)(w0 + s * p.tdw) < (unsigned)p.gW) mask |= 1u << (16 + s);
                    conv_mask[j] = m < p.M ? mask : 0u;
                    conv_base[j] = (((n * p.gH + h0) * p.gW + w0) * p.gC) * 2;
                } else {
                    conv_pix[j] = n * p.gH * p.gW * p.gC;
                    conv_h0[j] = m < p.M ? h0 : -(1 << 28);  // invalid rows never hit the image
                    conv_w0[j] = w0;
                }
                da.voff[j] = 0;
            } else if constexpr (C::A_KC) {
                // A row-major: tile row = m, chunk c covers k = 8c .. 8c+7 of the current K tile
                const bool ok = m0 + row < p.M;
                da.voff[j] = ok ? (uint32_t)(row * p.lda * 2 + c * 16) : kOob;
            } else {
                // A column-major: LDS row = k, chunk c covers m = m0 + 8c .. +7
                const bool ok = m0 + 8 * c < p.M;
                da.voff[j] = ok ? (uint32_t)(row * p.lda * 2 + c * 16) : kOob;
            }
        }
        // Operand B
#pragma unroll
        for (int j = 0; j < TB::IPW; ++j) {
            const int q = j * C::NL + wave;
            const int row = TB::row_of(q, lane);
            const int c = TB::logical_chunk(q, lane);
            if constexpr (C::B_KC) {
                // B column-major (N x K storage): tile row = n
                const bool ok = n0 + row < p.N;
                db.voff[j] = ok ? (uint32_t)(row * p.ldb * 2 + c * 16) : kOob;
            } else {
                // B row-major (K x N storage): LDS row = k, chunk c covers n = n0 + 8c .. +7
                const bool ok = n0 + 8 * c < p.N;
                db.voff[j] = ok ? (uint32_t)(row * p.ldb * 2 + c * 16) : kOob;
                if constexpr (C::DGRAD && !kUniformTap) dg_col[j] = ok ? (uint32_t)(c * 16) : kOob;
                if constexpr (C::WGRAD) {
                    // column n0 + 8c = (tap, channel) of the filter gradient; a
                    // chunk never straddles taps since Cin % 8 == 0
                    const int nc = (int)(ok ? n0 + 8 * c : 0);
                    const int tap = nc / p.Cin, ch = nc - tap * p.Cin;
                    const int r = tap / p.S, sc = tap - r * p.S;
                    wg_rd[j] = ok ? r * p.dh : -(1 << 28);
                    wg_sd[j] = sc * p.dw;
                    wg_c2[j] = ch * 2;
                }
            }
        }
    }

    __device__ __forceinline__ void setup_frag_offsets() {
        // K-contiguous: lane reads row (wave row + MI*i + lane%MI), logical chunk
        // NH*kk + lane/MI (the lane's 8 k of the k-step).  The swizzle depends on
        // row % 16 only, so it is the same for every fragment i.
        // M/N-contiguous (ds_read_b64_tr_b16, 4 k-rows x 16 columns per 16-lane
        // group g, lane i16 addressing k-row i16/4 and columns 4*(i16%4)..+3):
        //   32x32x16: group g covers k-rows 8*(g/2).. of the k-step and the
        //             16 columns 16*(g%2).. of a 32-column fragment;
        //   16x16x32: group g covers k-rows 8*g.. and the fragment's 16 columns.
        // The k-row's swizzle depends on bits 0, 1 and 3 of the row only, which
        // the k-step origin and the +4-row second read leave unchanged.
        const int g = lane >> 4, i16 = lane & 15;
        const int mn_rowpart = MI == 32 ? 8 * (g >> 1) + (i16 >> 2) : 8 * g + (i16 >> 2);
        const int mn_u = MI == 32 ? 2 * (g & 1) + ((i16 & 3) >> 1) : ((i16 & 3) >> 1);
        if constexpr (C::A_KC) {
            const int row = wm * C::WTM + (lane % MI);
            const int x = (lane / MI) ^ swz_k<TA::CPR>(row);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) fa_off[kk] = row * BK * 2 + (((NH * kk) ^ x) * 16);
        } else {
            const int mn_sa = swz_mn<TA::CPR>(mn_rowpart);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int cl = (wm * C::WTM) / 8 + (MI / 8) * i + mn_u;
                fa_off[i] = mn_rowpart * BM * 2 + ((cl ^ mn_sa) * 16) + 8 * (i16 & 1);
            }
        }
        if constexpr (C::B_KC) {
            const int row = wn * C::WTN + (lane % MI);
            const int x = (lane / MI) ^ swz_k<TB::CPR>(row);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) fb_off[kk] = row * BK * 2 + (((NH * kk) ^ x) * 16);
        } else {
            const int mn_sb = swz_mn<TB::CPR>(mn_rowpart);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int cl = (wn * C::WTN) / 8 + (MI / 8) * j + mn_u;
                fb_off[j] = mn_rowpart * BN * 2 + ((cl ^ mn_sb) * 16) + 8 * (i16 & 1);
            }
        }
    }

    // ---- global -> LDS: the loads of K tile t ---------------------------------
    // Wave instructions J0 .. J1-1 of operand OP (0: A, 1: B) of tile t into its
    // slot.  Masking is branch-free: a chunk past M/N was given an out-of-range
    // offset at setup; a chunk past K (the K tail, and every load of the
    // padding tiles t >= KT) is masked per lane here.  Because q = j*NW + wave,
    // a lane's swizzled K chunk is the same for all of its loads of one
    // operand, so one compare per tile does.
    template <int OP, int J0, int J1>
    __device__ __forceinline__ void issue_op(int t, IGC_LDS char* dst) {
        if constexpr (!LOADER) return;
        const int64_t k0 = kbase + (int64_t)t * BK;
        IGC_LDS char* sa = dst;
        IGC_LDS char* sb = dst;
        // valid K elements left from this tile on, clamped to [0, BK] on the
        // scalar side so the per-lane masks below are 32-bit compares
        const int64_t krem64 = kend - k0;
        const int krem = krem64 <= 0 ? 0 : (krem64 >= BK ? BK : (int)krem64);
        // ---- A
        if constexpr (OP == 0 && J1 > J0) {
            if constexpr (C::GATHER_A) {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc_u(p.A);
                // K index k = ((r*S + s) * gC + c): filter tap (r, s), channel c.
                // This lane's chunk is the same logical chunk for all its loads.
                int r, s, cin;
                if constexpr (kUniformTap) {
                    // the whole tile lies in one tap: scalar split of the tile index
                    const uint32_t tg = (uint32_t)(k0 / BK);
                    const uint32_t tap = fastdiv(tg, (uint32_t)p.tpt, p.tpt_magic);
                    const uint32_t rr = fastdiv(tap, (uint32_t)p.S, p.s_magic);
                    r = (int)rr;
                    s = (int)(tap - rr * (uint32_t)p.S);
                    cin = (int)(tg - tap * (uint32_t)p.tpt) * BK + 8 * ca_lane;
                } else {
                    const uint32_t kg = (uint32_t)k0 + 8u * (uint32_t)ca_lane;
                    const uint32_t tap = fastdiv(kg, (uint32_t)p.gC, p.cin_magic);
                    const uint32_t rr = fastdiv(tap, (uint32_t)p.S, p.s_magic);
                    r = (int)rr;
                    s = (int)(tap - rr * (uint32_t)p.S);
                    cin = (int)(kg - tap * (uint32_t)p.gC);
                }
                const bool kok = 8 * ca_lane < krem;
                if constexpr (kConvMasks) {
                    // tap (r, s) of a row is in the image iff both its mask bits are set
                    const uint32_t need = (1u << (r & 15)) | (1u << (16 + (s & 15)));
                    const int toff = ((r * p.tdh * p.gW + s * p.tdw) * p.gC + cin) * 2;
                    static_for<J0, J1>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = J;
                        const int q = j * C::NL + wave;
                        const bool ok = kok && (conv_mask[j] & need) == need;
                        dma16(rs, sa + q * 1024, ok ? (uint32_t)(conv_base[j] + toff) : kOob);
                    });
                } else {
                    const int dhr = r * p.tdh, dws = s * p.tdw;
                    static_for<J0, J1>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = J;
                        const int q = j * C::NL + wave;
                        int h = conv_h0[j] + dhr;
                        int w = conv_w0[j] + dws;
                        bool ok = kok;
                        if constexpr (C::DGRAD) {
                            // the tap lands on an output row/column only at multiples of the stride
                            const int hq = (int)fastdiv((uint32_t)(h < 0 ? 0 : h), (uint32_t)p.gsh, p.gsh_magic);
                            const int wq = (int)fastdiv((uint32_t)(w < 0 ? 0 : w), (uint32_t)p.gsw, p.gsw_magic);
                            ok = ok && h >= 0 && w >= 0 && hq * p.gsh == h && wq * p.gsw == w;
                            h = hq;
                            w = wq;
                        }
                        ok = ok && (unsigned)h < (unsigned)p.gH && (unsigned)w < (unsigned)p.gW;
                        // unsigned arithmetic: rows past M carry a huge negative h and are discarded
                        const uint32_t off =
                            ((uint32_t)conv_pix[j] + ((uint32_t)h * (uint32_t)p.gW + (uint32_t)w) * (uint32_t)p.gC +
                             (uint32_t)cin) * 2u;
                        dma16(rs, sa + q * 1024, ok ? off : kOob);
                    });
                }
            } else if constexpr (C::A_KC) {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc_u((const char*)p.A + (m0 * p.lda + k0) * 2);
                const bool kout = 8 * ca_lane >= krem;
                static_for<J0, J1>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = J;
                    dma16(rs, sa + (j * C::NL + wave) * 1024, kout ? kOob : da.voff[j]);
                });
            } else {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc_u((const char*)p.A + (k0 * p.lda + m0) * 2);
                static_for<J0, J1>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = J;
                    const int q = j * C::NL + wave;
                    dma16(rs, sa + q * 1024, TA::row_of(q, lane) >= krem ? kOob : da.voff[j]);
                });
            }
        }
        // ---- B
        if constexpr (OP == 1 && J1 > J0) {
            constexpr int B0 = J0, B1 = J1;
            if constexpr (C::B_KC) {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc_u((const char*)p.B + (n0 * p.ldb + k0) * 2);
                const bool kout = 8 * cb_lane >= krem;
                static_for<B0, B1>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = J;
                    dma16(rs, sb + (j * C::NL + wave) * 1024, kout ? kOob : db.voff[j]);
                });
            } else if constexpr (C::DGRAD) {
                // K row k0 + i = (tap, output channel kc) reads filter row kc*R*S + tap
                const int RS = p.R * p.S;
                if constexpr (kUniformTap) {
                    // the tile lies in one tap: rows kc0 .. kc0+BK-1 are ldb = R*S*Cin apart
                    // 32-bit scalar arithmetic (the filter spans < 2^31 bytes), made explicitly
                    // uniform: a base computed in vector registers would force a waterfall loop
                    // around every load of the tile
                    const uint32_t tap = fastdiv((uint32_t)k0, (uint32_t)p.gC, p.cin_magic);
                    const uint32_t kc0 = (uint32_t)k0 - tap * (uint32_t)p.gC;
                    const uint32_t base = __builtin_amdgcn_readfirstlane(
                        ((kc0 * (uint32_t)RS + tap) * (uint32_t)p.N + (uint32_t)n0) * 2u);
                    const __amdgpu_buffer_rsrc_t rs = make_rsrc_u((const char*)p.B + base);
                    static_for<B0, B1>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = J;
                        const int q = j * C::NL + wave;
                        dma16(rs, sb + q * 1024, TB::row_of(q, lane) >= krem ? kOob : db.voff[j]);
                    });
                } else {
                    const __amdgpu_buffer_rsrc_t rs = make_rsrc_u((const char*)p.B + n0 * 2);
                    static_for<B0, B1>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = J;
                        const int q = j * C::NL + wave;
                        const int row = TB::row_of(q, lane);
                        const uint32_t kg = (uint32_t)k0 + (uint32_t)row;
                        const uint32_t tap = fastdiv(kg, (uint32_t)p.gC, p.cin_magic);
                        const uint32_t kc = kg - tap * (uint32_t)p.gC;
                        const uint32_t off = (kc * (uint32_t)RS + tap) * (uint32_t)p.N * 2u + dg_col[j];
                        dma16(rs, sb + q * 1024, (row >= krem || dg_col[j] == kOob) ? kOob : off);
                    });
                }
            } else if constexpr (C::WGRAD) {
                // K row k0 + i = output pixel (n, p, q); its window's tap (r, s)
                // reads x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][channel]
                const __amdgpu_buffer_rsrc_t rs = make_rsrc_u(p.B);
                const uint32_t PQ = (uint32_t)(p.P * p.Q);
                static_for<B0, B1>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = J;
                    const int q = j * C::NL + wave;
                    const int row = TB::row_of(q, lane);
                    const uint32_t pix = (uint32_t)k0 + (uint32_t)row;
                    const uint32_t n = fastdiv(pix, PQ, p.pq_magic);
                    const uint32_t pq = pix - n * PQ;
                    const uint32_t pp = fastdiv(pq, (uint32_t)p.Q, p.q_magic);
                    const int qq = (int)(pq - pp * (uint32_t)p.Q);
                    const int h = (int)pp * p.sh - p.ph + wg_rd[j];
                    const int w = qq * p.sw - p.pw + wg_sd[j];
                    const bool ok = row < krem && (unsigned)h < (unsigned)p.H && (unsigned)w < (unsigned)p.W;
                    const uint32_t off =
                        ((n * (uint32_t)p.H + (uint32_t)h) * (uint32_t)p.W + (uint32_t)w) * (uint32_t)p.Cin * 2u +
                        (uint32_t)wg_c2[j];
                    dma16(rs, sb + q * 1024, ok ? off : kOob);
                });
            } else {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc_u((const char*)p.B + (k0 * p.ldb + n0) * 2);
                static_for<B0, B1>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = J;
                    const int q = j * C::NL + wave;
                    dma16(rs, sb + q * 1024, TB::row_of(q, lane) >= krem ? kOob : db.voff[j]);
                });
            }
        }
    }

    template <int OP>
    static constexpr int ipw() { return OP == 0 ? TA::IPW : TB::IPW; }

    // All loads of tile t.  Tiles t >= KT are padding tiles: every load is out
    // of range, the slot fills with zeros and the MFMAs on it add exact zeros.
    __device__ __forceinline__ void issue(int t, IGC_LDS char* sa, IGC_LDS char* sb) {
        issue_op<0, 0, TA::IPW>(t, sa);
        issue_op<1, 0, TB::IPW>(t, sb);
    }

    // Part PART of NPARTS of the loads of two ring units: operand OP1 of tile
    // t1 into d1, then operand OP2 of tile t2 into d2 (numbered in that order).
    template <int PART, int NPARTS, int OP1, int OP2>
    __device__ __forceinline__ void issue_units_part(int t1, IGC_LDS char* d1, int t2, IGC_LDS char* d2) {
        constexpr int N1 = ipw<OP1>(), N = N1 + ipw<OP2>();
        constexpr int J0 = PART * N / NPARTS, J1 = (PART + 1) * N / NPARTS;
        issue_op<OP1, (J0 < N1 ? J0 : N1), (J1 < N1 ? J1 : N1)>(t1, d1);
        issue_op<OP2, (J0 > N1 ? J0 - N1 : 0), (J1 > N1 ? J1 - N1 : 0)>(t2, d2);
    }

    // After this wave's loads of K tile t have landed and before the barrier:
    // when K % 8 != 0, the chunk straddling K holds elements k >= K read from
    // beyond the row's end; the lane that fetched it zeroes them.
    __device__ __forceinline__ void fixup_ragged_k(int t, IGC_LDS char* sa, IGC_LDS char* sb) {
        if constexpr (!kRagged || !LOADER) return;
        const int64_t k0 = kbase + (int64_t)t * BK;
        if (!p.k_ragged8 || k0 + BK <= p.K) return;
        // the only chunk that straddles K is the one starting at k0 + 8*cs
        const int cs = (int)((p.K - k0) >> 3);
        const int keep = (int)((p.K - k0) & 7);  // elements of that chunk below K
        // bytes of the 16-byte chunk to keep: the first 2*keep
        const uint32_t m0w = keep >= 2 ? 0xffffffffu : (keep == 1 ? 0x0000ffffu : 0u);
        const uint32_t m1w = keep >= 4 ? 0xffffffffu : (keep == 3 ? 0x0000ffffu : 0u);
        const uint32_t m2w = keep >= 6 ? 0xffffffffu : (keep == 5 ? 0x0000ffffu : 0u);
        const uint32_t m3w = keep == 7 ? 0x0000ffffu : 0u;
        auto fix = [&](IGC_LDS char* region, int q, int c) __attribute__((always_inline)) {
            if (c == cs) {
                typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
                IGC_LDS u32x4_t* e = (IGC_LDS u32x4_t*)(region + q * 1024 + lane * 16);
                u32x4_t v = *e;
                v[0] &= m0w;
                v[1] &= m1w;
                v[2] &= m2w;
                v[3] &= m3w;
                *e = v;
            }
        };
        if constexpr (C::A_KC && !C::GATHER_A) {
#pragma unroll
            for (int j = 0; j < TA::IPW; ++j) {
                const int q = j * C::NL + wave;
                fix(sa, q, TA::logical_chunk(q, lane));
            }
        }
        if constexpr (C::B_KC) {
#pragma unroll
            for (int j = 0; j < TB::IPW; ++j) {
                const int q = j * C::NL + wave;
                fix(sb, q, TB::logical_chunk(q, lane));
            }
        }
    }

    // ---- LDS -> registers: fragments of one MFMA k-step ----------------------
    // Order: A fragment 0, every B fragment, then the other A fragments -- the
    // order in which the MFMAs of the k-step consume them.
    __device__ __forceinline__ void read_a(const IGC_LDS char* sa, int kk, int i, i16x8_t& f) {
        if constexpr (C::A_KC) {
            f = *(const IGC_LDS i16x8_t*)(sa + fa_off[kk] + i * MI * BK * 2);
        } else {
            const IGC_LDS char* a0 = sa + fa_off[i] + (KS * kk) * BM * 2;
            i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((IGC_LDS i16x4_t*)a0);
            i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((IGC_LDS i16x4_t*)(a0 + 4 * BM * 2));
            f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    __device__ __forceinline__ void read_b(const IGC_LDS char* sb, int kk, int j, i16x8_t& f) {
        if constexpr (C::B_KC) {
            f = *(const IGC_LDS i16x8_t*)(sb + fb_off[kk] + j * MI * BK * 2);
        } else {
            const IGC_LDS char* b0 = sb + fb_off[j] + (KS * kk) * BN * 2;
            i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((IGC_LDS i16x4_t*)b0);
            i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((IGC_LDS i16x4_t*)(b0 + 4 * BN * 2));
            f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    __device__ __forceinline__ void read_frags(const IGC_LDS char* sa, const IGC_LDS char* sb, int kk,
                                               i16x8_t (&fa)[FM], i16x8_t (&fb)[FN]) {
        read_a(sa, kk, 0, fa[0]);
#pragma unroll
        for (int j = 0; j < FN; ++j) read_b(sb, kk, j, fb[j]);
#pragma unroll
        for (int i = 1; i < FM; ++i) read_a(sa, kk, i, fa[i]);
    }
    // LDS read instructions of one k-step
    static constexpr int DS_READS = FM * (C::A_KC ? 1 : 2) + FN * (C::B_KC ? 1 : 2);

    __device__ __forceinline__ static void mma(Acc (&acc)[FM][FN], const i16x8_t (&fa)[FM], const i16x8_t (&fb)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma<C::FP16>(fb[j], fa[i], acc[i][j]);
    }

    // Wait until at most n later K tiles of this wave's loads are still in
    // flight (n in [0, D-2]); loads complete in issue order, so the oldest
    // outstanding tile has then landed.
    template <int NMAX>
    __device__ __forceinline__ static void wait_tiles(int n) {
        if constexpr (NMAX <= 0) {
            wait_vmcnt<0>();
        } else {
            if (n >= NMAX) {
                wait_vmcnt<NMAX * C::LPT>();
            } else {
                wait_tiles<NMAX - 1>(n);
            }
        }
    }

    // ---- stream-K partial tiles ----------------------------------------------
    // A partial tile is kept in lane order: 16-byte piece c of accumulator
    // block (i, j) of wave w lies at float4 index ((w*FM + i)*FN + j)*NQ + c,
    // times 64, plus the lane, so every store and load is one coalesced 1 KB
    // wave access.
    static constexpr int NQ = (int)(sizeof(Acc) / 16);
    static_assert(C::NT / 64 * FM * FN * NQ * 64 * 4 == BM * BN, "partial tile holds BM x BN floats");

    // Partial tiles and flags move with system-coherent buffer accesses (SC0 and
    // SC1 set: stores write through to memory, loads do not hit stale cache
    // lines), so workgroups on different XCDs exchange them without flushing
    // or invalidating the caches other workgroups are using.
    static constexpr int kCoherent = 1 | 16;             // SC0 | SC1
    static constexpr int kCoherentVolatile = kCoherent | (1 << 31);

    // Writes the partial tile, waits until this wave's stores are complete,
    // and (once every wave is there) raises the flag to 1.  `raise` false is
    // the test hook that leaves one flag down.
    __device__ __forceinline__ void sk_publish(const Acc (&acc)[FM][FN], float* part, int* flag, bool raise) {
        typedef __attribute__((ext_vector_type(4))) int i32x4_t;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(part);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const f32x4_t v{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
                    const int off = ((((wave * FM + i) * FN + j) * NQ + c) * 64 + lane) * 16;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), rs, off, 0, kCoherent);
                }
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0 && raise) __builtin_amdgcn_raw_buffer_store_b32(1, make_rsrc(flag), 0, 0, kCoherent);
    }

    // Waits (bounded: at most `spins` polls) for a lower workgroup's flag and,
    // if it rose, adds its partial tile.  Thread 0 polls; its verdict reaches
    // every wave through the first word of the drained ring (`bcast`), so all
    // waves agree.  Returns false if the wait gave up.  Every wave must call
    // it, after its K loop.
    __device__ __forceinline__ bool sk_collect(Acc (&acc)[FM][FN], const float* part, int* flag, int spins,
                                               IGC_LDS int* bcast) {
        __syncthreads();  // every wave is done reading the ring (and an earlier verdict)
        if (threadIdx.x == 0) {
            const __amdgpu_buffer_rsrc_t rf = make_rsrc(flag);
            int up = 0;
            for (int n = 0; n < spins && !up; ++n) {
                up = __builtin_amdgcn_raw_buffer_load_b32(rf, 0, 0, kCoherentVolatile) == 1;
                if (!up) __builtin_amdgcn_s_sleep(2);
            }
            *(volatile IGC_LDS int*)bcast = up;
        }
        __syncthreads();
        const bool up = *(volatile IGC_LDS int*)bcast != 0;
        if (!up) return false;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(part);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const int off = ((((wave * FM + i) * FN + j) * NQ + c) * 64 + lane) * 16;
                    const f32x4_t v = __builtin_bit_cast(
                        f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherentVolatile));
                    acc[i][j][4 * c] += v[0];
                    acc[i][j][4 * c + 1] += v[1];
                    acc[i][j][4 * c + 2] += v[2];
                    acc[i][j][4 * c + 3] += v[3];
                }
        return true;
    }

    // ---- epilogue: accumulators -> C ---------------------------------------
    // Lane l holds, of block (i, j), row MI*i + l%MI and, in accumulators
    // 4g..4g+3, the 4 consecutive columns MI*j + 4*NH*g + 4*(l/MI) + 0..3.
    __device__ __forceinline__ void store(const Acc (&acc)[FM][FN], void* dst, int64_t ldc, int kind,
                                          bool vec_ok) {
        constexpr int NG = MI == 32 ? 4 : 1;  // groups of 4 accumulators per block
        const bool full = vec_ok && (m0 + BM <= p.M) && (n0 + BN <= p.N);
        const int64_t mrow = m0 + wm * C::WTM + (lane % MI);
        const int64_t ncol = n0 + wn * C::WTN + 4 * (lane / MI);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t m = mrow + MI * i;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                // one block at a time: only its accumulators move to VGPRs at once
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int64_t n = ncol + MI * j + 4 * NH * g;
                    const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                    const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                    const int64_t off = m * ldc + n;
                    if (full) {
                        if (kind == OUT_F32) {
                            *(f32x4_t*)((float*)dst + off) = f32x4_t{v0, v1, v2, v3};
                        } else if (kind == OUT_BF16) {
                            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
                            *(bf16x4_t*)((__bf16*)dst + off) = bf16x4_t{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                        } else {
                            typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
                            *(f16x4_t*)((_Float16*)dst + off) =
                                f16x4_t{(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
                        }
                    } else if (m < p.M) {
                        const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (n + e < p.N) {
                                if (kind == OUT_F32)
                                    ((float*)dst)[off + e] = v[e];
                                else if (kind == OUT_BF16)
                                    ((__bf16*)dst)[off + e] = (__bf16)v[e];
                                else
                                    ((_Float16*)dst)[off + e] = (_Float16)v[e];
                            }
                        }
                    }
                }
            }
        }
    }
};

}  // namespace igc

namespace igc {

// Compiler-level memory ordering point (emits no instruction).  The hardware
// ordering comes from the explicit s_waitcnt and s_barrier around it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Every wave has drained its own LDS reads (and, before that, waited for its
// own direct-to-LDS loads); then the workgroup meets.
__device__ __forceinline__ void ring_barrier() {
    wait_lgkmcnt0();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Workgroup i is dispatched to XCD i % 8, and each XCD has its own L2:
// xcd_order gives every XCD a contiguous range of the `count` work ids.
__device__ __forceinline__ int xcd_order(int wg, int count) {
    constexpr int kXcds = 8;
    const int q = count / kXcds, r = count % kXcds, x = wg % kXcds, i = wg / kXcds;
    return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Tile id -> (tile_m, tile_n), walking GROUP_M tiles down M at a time, so that
// a contiguous range of ids (the tiles resident on one XCD) shares A rows and
// B columns in that XCD's L2.
__device__ __forceinline__ void group_coords(int id, int tiles_m, int tiles_n, int kGroupM, int& tm, int& tn) {
    const int group = kGroupM * tiles_n;
    const int g = id / group;
    const int first_m = g * kGroupM;
    const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
    const int in = id - g * group;
    tm = first_m + in % gm;
    tn = in / gm;
}

// blockIdx -> (tile_m, tile_n) for a grid of one workgroup per tile.
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int kGroupM, int& tm, int& tn) {
    group_coords(xcd_order(wg, tiles_m * tiles_n), tiles_m, tiles_n, kGroupM, tm, tn);
}

// Scheduling template for one k-step region: NM MFMAs with ND LDS reads and
// NV global->LDS loads spread between them, so the reads and loads issue while
// earlier MFMAs execute instead of in a burst ahead of them.
template <int NM, int ND, int NV>
__device__ __forceinline__ void interleave() {
    constexpr int kMfma = 0x008, kDsRead = 0x100, kVmemRead = 0x020;
    static_for<0, NM>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = I;
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        constexpr int d0 = i * ND / NM, d1 = (i + 1) * ND / NM;
        if constexpr (d1 > d0) __builtin_amdgcn_sched_group_barrier(kDsRead, d1 - d0, 0);
        constexpr int v0 = i * NV / NM, v1 = (i + 1) * NV / NM;
        if constexpr (v1 > v0) __builtin_amdgcn_sched_group_barrier(kVmemRead, v1 - v0, 0);
    });
}

// LDS slot S of the ring of configuration C: one __shared__ array per slot,
// so every slot is a distinct object to the compiler.
template <class C, int S>
__device__ __forceinline__ IGC_LDS char* slot() {
    __shared__ __attribute__((aligned(1024))) char buf[C::template slot_bytes<S>()];
    return (IGC_LDS char*)buf;
}
// Slots of operand A and B of the u-th tile of an unrolled period.
template <class C, int u>
__device__ __forceinline__ IGC_LDS char* slot_a() { return slot<C, Ring::slot_of(C::U, 2 * u)>(); }
template <class C, int u>
__device__ __forceinline__ IGC_LDS char* slot_b() { return slot<C, Ring::slot_of(C::U, 2 * u + 1)>(); }

// Whole R-byte pieces the ring's slots hold when each piece lies inside one slot.
template <class C, int R, int S = 0>
constexpr int stage_pieces() {
    if constexpr (S >= C::U)
        return 0;
    else
        return C::template slot_bytes<S>() / R + stage_pieces<C, R, S + 1>();
}
// Piece w of that packing (slots in order).
template <class C, int R, int S = 0>
__device__ __forceinline__ IGC_LDS char* stage_piece(int w) {
    if constexpr (S >= C::U) {
        return nullptr;
    } else {
        constexpr int n = C::template slot_bytes<S>() / R;
        if (w < n) return slot<C, S>() + w * R;
        return stage_piece<C, R, S + 1>(w - n);
    }
}

// Staged-row swizzle, in 8-byte slots: slot s of row r of a staged row of
// `slots` slots (16: 128 bytes, 32: 256 bytes) is stored at s ^ f(r).  A
// 64-bit staging write puts 16 (or 32) consecutive rows at one column of an
// MFMA block, every row starting on the same bank, so f must spread them:
// f(r) differs for any 16 consecutive rows modulo 16 slots (16 lanes per
// clock on 32 banks of 4 bytes, the model under which the earlier map's
// measured conflicts appear) and, for any 32 lanes, lands them on distinct
// 8-byte units of a 256-byte cycle (32 lanes per clock on 64 banks).  The map
// XORs one value into both halves of a 16-byte chunk, so a 16-byte read finds
// a logical chunk whole in one physical chunk, halves swapped when f is odd.
IGC_HD inline int stage_slot(int row, int slot, int slots) {
    const int f = slots >= 32 ? (((row & 15) << 1) | ((row >> 3) & 1)) ^ ((row >> 4) & 1)
                              : (row & 15) ^ ((row >> 4) & 1);
    return slot ^ f;
}

// Blocks I0 .. I0+NI-1 (MFMA block rows) of a wave's sub-tile, as ESZ-byte
// elements: written into the wave's LDS piece `reg` (row-major, swizzled
// chunks), read back 16 bytes per lane and stored as whole row segments.
template <class C, int ESZ, int I0, int NI, class ML>
__device__ __forceinline__ void stage_rows(ML& ml, const typename C::Acc (&acc)[C::FM][C::FN], IGC_LDS char* reg,
                                           void* dst, int64_t ldc, int kind) {
    constexpr int MI = C::MI, NH = C::NH, NG = MI == 32 ? 4 : 1;
    constexpr int RB = C::WTN * ESZ;  // bytes per staged row
    constexpr int CPR = RB / 16;      // 16-byte chunks per staged row
    static_assert(ESZ == 2 && (CPR == 8 || CPR == 16), "16-bit rows of 128 or 256 bytes");
    const int lane = ml.lane;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int row = MI * i + lane % MI;
                const int byte = (MI * j + 4 * NH * g + 4 * (lane / MI)) * ESZ;
                IGC_LDS char* a = reg + row * RB + (stage_slot(row, byte >> 3, 2 * CPR) << 3);
                const float v0 = acc[I0 + i][j][4 * g + 0], v1 = acc[I0 + i][j][4 * g + 1];
                const float v2 = acc[I0 + i][j][4 * g + 2], v3 = acc[I0 + i][j][4 * g + 3];
                if (kind == OUT_BF16) {
                    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
                    *(IGC_LDS bf16x4_t*)a = bf16x4_t{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                } else {
                    typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
                    *(IGC_LDS f16x4_t*)a = f16x4_t{(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
                }
            }
    // the wave's own writes, read back by other lanes of the same wave
    wait_lgkmcnt0();
    compiler_fence();
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
    constexpr int RPI = 64 / CPR;  // staged rows per read instruction
    const int64_t gm0 = ml.m0 + ml.wm * C::WTM + MI * I0, gn0 = ml.n0 + ml.wn * C::WTN;
#pragma unroll
    for (int q = 0; q < NI * MI / RPI; ++q) {
        const int row = q * RPI + lane / CPR, c = lane % CPR;
        // slots 2c and 2c+1 stay one 16-byte chunk (the map XORs one value into both), in swapped order
        // when slot 2c lands odd
        const int p0 = stage_slot(row, 2 * c, 2 * CPR);
        u32x4_t v = *(const IGC_LDS u32x4_t*)(reg + row * RB + ((p0 >> 1) << 4));
        if (p0 & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
        *(u32x4_t*)((char*)dst + ((gm0 + row) * ldc + gn0) * ESZ + c * 16) = v;
    }
    // reads done before the piece is written again
    wait_lgkmcnt0();
    compiler_fence();
}

// Output epilogue.  A full tile goes through LDS: after the ring's last reads,
// each wave writes its WTM x WTN sub-tile, converted, into a private piece of
// the drained ring, reads it back 16 bytes per lane and stores whole row
// segments, so every store instruction writes runs of consecutive addresses
// (whole 128-byte lines) instead of 8- or 16-byte pieces of 16 or 32 rows,
// which the memory system retires far faster.  Edge tiles and fp32 output
// store straight from the accumulators (staging fp32 as two passes of
// stage_rows<C, 4, ...> raised the register pressure of the whole kernel until
// its K loop spilled).  Must be called by every wave of the workgroup (it has a
// barrier when it stages), with no loads into the ring outstanding.
template <class C, class ML>
__device__ __forceinline__ void store_tile(ML& ml, const typename C::Acc (&acc)[C::FM][C::FN], void* dst,
                                           int64_t ldc, int kind, bool vec_ok) {
    constexpr int R = C::WTM * C::WTN * 2;  // bytes of one wave's LDS piece
    if constexpr (stage_pieces<C, R>() >= C::NW && C::WTN * 2 >= 128) {
        const bool full = vec_ok && kind != OUT_F32 && ml.m0 + C::BM <= ml.p.M && ml.n0 + C::BN <= ml.p.N;
        if (full) {
            ring_barrier();  // every wave has finished reading the ring
            stage_rows<C, 2, 0, C::FM>(ml, acc, stage_piece<C, R>(ml.wave), dst, ldc, kind);
            return;
        }
    }
    ml.store(acc, dst, ldc, kind, vec_ok);
}

// Per-stage counters of the SYNC 1 ring: ready[s] at [s], free[s] at [D + s].
// A stage is filled once per pass around the ring, so after pass n (tiles
// n*D + s) ready[s] reaches NL*(n+1) (each loading wave adds one when its own
// loads into the stage have landed) and free[s] reaches NW*(n+1) (each wave
// adds one when its reads of the stage have drained).
template <class C>
__device__ __forceinline__ IGC_LDS int* stage_counters() {
    __shared__ int ctr[2 * C::D];
    return (IGC_LDS int*)ctr;
}

// The counter operations are written as single instruction sequences: a
// C-level poll loop (and the lane-0 branch of the atomic) splits the K loop
// into many basic blocks, and across them the compiler no longer keeps the
// accumulators in place (it renames and copies them, and the compute-only
// copy of the loop spills).

// One wave adds one to a counter: lane 0 alone issues the LDS atomic.
__device__ __forceinline__ void count_up(IGC_LDS int* c) {
    uint64_t save;
    uint32_t one;
    asm volatile(
        "s_mov_b64 %[save], exec\n\t"
        "s_mov_b64 exec, 1\n\t"
        "v_mov_b32 %[one], 1\n\t"
        "ds_add_u32 %[a], %[one]\n\t"
        "s_mov_b64 exec, %[save]"
        : [save] "=&s"(save), [one] "=&v"(one)
        : [a] "v"((uint32_t)(uintptr_t)c)
        : "memory");
}

// Waits until *c >= target, polling with a short sleep between reads; the
// read is waited for inside the same sequence.  Bounded: after `limit` polls
// it gives up and returns true (a protocol mistake then shows as a wrong,
// reported result rather than a hung GPU).
__device__ __forceinline__ bool wait_count(IGC_LDS int* c, int target, int limit = 1 << 22) {
    uint32_t v;
    int seen, n;
    asm volatile(
        "s_mov_b32 %[n], %[lim]\n"
        "1:\n\t"
        "ds_read_b32 %[v], %[a]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_readfirstlane_b32 %[seen], %[v]\n\t"
        "s_cmp_ge_i32 %[seen], %[t]\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_sub_u32 %[n], %[n], 1\n\t"
        "s_cmp_eq_u32 %[n], 0\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_sleep 1\n\t"
        "s_branch 1b\n"
        "2:"
        : [v] "=&v"(v), [seen] "=&s"(seen), [n] "=&s"(n)
        : [a] "v"((uint32_t)(uintptr_t)c), [t] "s"(target), [lim] "s"(limit)
        : "memory", "scc");
    return seen < target;
}

// The K range [kbase, kend) of one output tile: setup, the K loop of variant
// V, then epi(ml, acc) with the accumulators.
template <class C, int V, bool LOADER, class Epi>
__device__ __forceinline__ void run_tile_as(const Params p, int tm, int tn, int64_t kbase, int64_t kend, Epi&& epi);

template <class C, int V, class Epi>
__device__ __forceinline__ void run_tile(const Params p, int tm, int tn, int64_t kbase, int64_t kend, Epi&& epi) {
    if constexpr (C::NL == C::NW) {
        run_tile_as<C, V, true>(p, tm, tn, kbase, kend, epi);
    } else {
        // loading and compute-only waves run separately compiled copies of the
        // same loop (identical barrier sequences), so neither has a branch in it
        if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < C::NL)
            run_tile_as<C, V, true>(p, tm, tn, kbase, kend, epi);
        else
            run_tile_as<C, V, false>(p, tm, tn, kbase, kend, epi);
    }
}

template <class C, int V, bool LOADER, class Epi>
__device__ __forceinline__ void run_tile_as(const Params p, int tm, int tn, int64_t kbase, int64_t kend, Epi&& epi) {
    using ML = Mainloop<C, V, LOADER>;
    constexpr int D = C::D, KK = C::KK, FM = C::FM, FN = C::FN, U = C::U, P = C::P;
    // A loading wave shares its SIMD with a compute-only wave; issuing its
    // instructions first keeps the loads of whole-stage rings going out on
    // time (the compute-only wave's MFMAs fill the gaps).  Measured on the
    // 4-stage 32-deep ring: 1.5% off the GEMM and 3% off the conv (the
    // opposite priority costs 13%); on the 2.5-stage ring, whose refills are
    // already spread through the MFMAs, it slowed the conv by 30%.
    if constexpr (LOADER && C::NL != C::NW && C::HALF == 0) __builtin_amdgcn_s_setprio(2);
    ML ml(p, (int64_t)tm * C::BM, (int64_t)tn * C::BN, kbase, kend);
    const int KT = ml.KT, KTp = ml.KTp;

    typename C::Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = typename C::Acc{};
    // Two fragment register sets: k-step kk of the u-th tile of a period uses
    // set (u*KK + kk) % 2, while the next k-step's fragments load into the other.
    i16x8_t fa[2][FM], fb[2][FN];

    // The accumulators are never updated under a branch inside a loop: every
    // K tile of a loop runs the same MFMA sequence, so no copies of them are
    // needed (the guarded tiles of a partial last period follow the loop).
    constexpr int NMF = FM * FN;
    constexpr int DSR = ML::DS_READS;
    if constexpr (C::SPREAD) {
        // ---- operand-slot ring (ring.hpp): unit s = operand s%2 of tile s/2 in
        // slot s % U.  Prologue: units 0 .. U-3; during tile t the units
        // 2t+U-2 and 2t+U-1 (the slots of tile t-1, freed by the barrier that
        // made tile t ready) are refilled by loads spread over its k-steps.
        // SYNC 1 replaces each barrier by the stage counters: every wave marks
        // tile t's stage free and (loading waves) tile t+1's stage ready, then
        // waits for t+1 to be ready; a loading wave waits for a stage to be
        // free only before refilling it, so compute-only waves never wait for
        // another wave's reads.
        constexpr bool CTR = C::SYNC == 1;
        IGC_LDS int* ctr = nullptr;  // (the counters take LDS only in SYNC 1 instances)
        bool late = false;  // a counter wait gave up
        if constexpr (CTR) ctr = stage_counters<C>();
        if constexpr (CTR) {
            if (threadIdx.x < 2 * D) ctr[threadIdx.x] = 0;
            __syncthreads();  // counters are zero before anyone counts (the previous item is done with them)
        }
        constexpr int WAITN = Ring::wait_loads(U, ML::template ipw<0>(), ML::template ipw<1>());
        static_for<0, U - 2>([&](auto S) __attribute__((always_inline)) {
            constexpr int s = S;
            ml.template issue_op<s % 2, 0, ML::template ipw<s % 2>()>(s / 2, slot<C, s>());
        });
        wait_vmcnt<WAITN>();
        ml.fixup_ragged_k(0, slot_a<C, 0>(), slot_b<C, 0>());
        if constexpr (CTR) {
            wait_lgkmcnt0();
            compiler_fence();
            if constexpr (LOADER) count_up(ctr + 0);  // tile 0 ready (stage 0, pass 0)
            late |= wait_count(ctr + 0, C::NL);
        } else {
            ring_barrier();
        }
        ml.read_frags(slot_a<C, 0>(), slot_b<C, 0>(), 0, fa[0], fb[0]);
        // Tile t0+u of a period (u a constant, so every slot is one).
        auto tile = [&](auto UU, const int t0) __attribute__((always_inline)) {
            constexpr int u = UU;
            const int t = t0 + u;
            // the two units refilled during tile t
            constexpr int s1 = 2 * u + U - 2, s2 = 2 * u + U - 1;
            constexpr int op1 = s1 % 2, op2 = s2 % 2;
            const int t1 = t + (U - 2 - op1) / 2, t2 = t + (U - 1 - op2) / 2;
            IGC_LDS char* d1 = slot<C, Ring::slot_of(U, s1)>();
            IGC_LDS char* d2 = slot<C, Ring::slot_of(U, s2)>();
            constexpr int p0 = (u * KK) & 1;  // fragment set of this tile's k-step 0
            if constexpr (CTR && LOADER) {
                // the refill goes into the stage of tile t-1 (pass (t-1)/D, P == D here): every
                // wave must be done reading it; nothing to wait for before tile 0
                constexpr int sf = (u + D - 1) % D;
                late |= wait_count(ctr + D + sf, C::NW * (t0 / D + (u >= 1 ? 1 : 0)));
            }
            // k-steps 0 .. KK-2: refill, read ahead, MFMA
            static_for<0, KK - 1>([&](auto KI) __attribute__((always_inline)) {
                constexpr int kk = KI;
                constexpr int pc = (p0 + kk) & 1, pn = pc ^ 1;
                ml.template issue_units_part<kk, KK, op1, op2>(t1, d1, t2, d2);
                ml.read_frags(slot_a<C, u>(), slot_b<C, u>(), kk + 1, fa[pn], fb[pn]);
                ML::mma(acc, fa[pc], fb[pc]);
                // the loads of part kk of issue_units_part (both units: LPT in all)
                interleave<NMF, DSR, (kk + 1) * C::LPT / KK - kk * C::LPT / KK>();
                __builtin_amdgcn_sched_barrier(0);
            });
            constexpr int pl = (p0 + KK - 1) & 1;  // set of the last k-step; the next tile's first uses pl^1
            ml.template issue_units_part<KK - 1, KK, op1, op2>(t1, d1, t2, d2);
            // ready(t+1) and free(t): the units newer than B(t+1) may stay in flight
            wait_vmcnt<WAITN>();
            ml.fixup_ragged_k(t + 1, slot_a<C, (u + 1) % P>(), slot_b<C, (u + 1) % P>());
            if constexpr (CTR) {
                wait_lgkmcnt0();  // this wave's reads of tile t have drained
                compiler_fence();
                constexpr int sr = (u + 1) % D;
                count_up(ctr + D + u);                    // tile t's stage free
                if constexpr (LOADER) count_up(ctr + sr);  // tile t+1's stage ready (own loads landed)
                late |= wait_count(ctr + sr, C::NL * (t0 / D + (u + 1 == D ? 1 : 0) + 1));
            } else {
                ring_barrier();
            }
            ml.read_frags(slot_a<C, (u + 1) % P>(), slot_b<C, (u + 1) % P>(), 0, fa[pl ^ 1], fb[pl ^ 1]);
            ML::mma(acc, fa[pl], fb[pl]);
            interleave<NMF, DSR, 0>();
            __builtin_amdgcn_sched_barrier(0);
        };
        // Whole periods in the loop; the tiles of a last, partial period run
        // after it, each under its own test (those past KT are skipped, though
        // the loads the last tiles issue for them still go out, as zeros).
        int t0 = 0;
        for (; t0 + P <= KT; t0 += P) static_for<0, P>([&](auto UU) __attribute__((always_inline)) { tile(UU, t0); });
        if (t0 < KT)
            static_for<0, P - 1>([&](auto UU) __attribute__((always_inline)) {
                if (t0 + (int)UU < KT) tile(UU, t0);
            });
        wait_vmcnt<0>();  // the loads past KT are still landing in free slots
        if constexpr (CTR) {
            if (late && (threadIdx.x & 63) == 0)
                __builtin_amdgcn_raw_buffer_store_b32(1, make_rsrc(p.err_word), 0, 0, 1 | 16);
        }
    } else if constexpr (D >= 2) {
        // ---- two stages, refilled in one burst right after the barrier
        static_for<0, D>([&](auto S) __attribute__((always_inline)) {
            if (S < KTp) ml.issue(S, slot_a<C, S>(), slot_b<C, S>());
        });
        ml.template wait_tiles<D - 1>(Ring::inflight_after(D, KTp, 0));
        ml.fixup_ragged_k(0, slot_a<C, 0>(), slot_b<C, 0>());
        ring_barrier();
        ml.read_frags(slot_a<C, 0>(), slot_b<C, 0>(), 0, fa[0], fb[0]);
        // ---- steady state, unrolled by D so every slot is a constant
        for (int t0 = 0; t0 < KTp; t0 += D) {
            static_for<0, D>([&](auto UU) __attribute__((always_inline)) {
                constexpr int u = UU;
                constexpr int un = (u + 1) % D;
                const int t = t0 + u;
                constexpr int p0 = (u * KK) & 1;  // fragment set of this tile's k-step 0
                static_for<0, KK - 1>([&](auto KI) __attribute__((always_inline)) {
                    constexpr int kk = KI;
                    constexpr int pc = (p0 + kk) & 1, pn = pc ^ 1;
                    ml.read_frags(slot_a<C, u>(), slot_b<C, u>(), kk + 1, fa[pn], fb[pn]);
                    ML::mma(acc, fa[pc], fb[pc]);
                    interleave<NMF, DSR, 0>();
                    __builtin_amdgcn_sched_barrier(0);  // k-steps stay in order: two fragment sets live
                });
                constexpr int pl = (p0 + KK - 1) & 1;
                // ready(t+1): own loads landed, then everyone; free(t): all reads of t done.
                // After the last tile this is a harmless extra barrier and read.
                ml.template wait_tiles<D - 2>(Ring::inflight_after(D, KTp, t + 1));
                ml.fixup_ragged_k(t + 1, slot_a<C, un>(), slot_b<C, un>());
                ring_barrier();
                if (t + D < KTp) ml.issue(t + D, slot_a<C, u>(), slot_b<C, u>());
                ml.read_frags(slot_a<C, un>(), slot_b<C, un>(), 0, fa[pl ^ 1], fb[pl ^ 1]);
                ML::mma(acc, fa[pl], fb[pl]);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    } else {
        // ---- D == 1: one slot, no overlap of loads with compute
        static_assert(D != 1 || KK % 2 == 0, "the unpipelined loop alternates fragment sets within a tile");
        IGC_LDS char* sa = slot_a<C, 0>();
        IGC_LDS char* sb = slot_b<C, 0>();
        if (KT > 0) ml.issue(0, sa, sb);
        wait_vmcnt<0>();
        ml.fixup_ragged_k(0, sa, sb);
        ring_barrier();
        ml.read_frags(sa, sb, 0, fa[0], fb[0]);
        for (int t = 0; t < KT; ++t) {
            static_for<0, KK - 1>([&](auto KI) __attribute__((always_inline)) {
                constexpr int kk = KI;
                ml.read_frags(sa, sb, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
                ML::mma(acc, fa[kk & 1], fb[kk & 1]);
                __builtin_amdgcn_sched_barrier(0);
            });
            ring_barrier();  // free: every wave has read tile t
            if (t + 1 < KT) ml.issue(t + 1, sa, sb);
            wait_vmcnt<0>();
            ml.fixup_ragged_k(t + 1, sa, sb);
            ring_barrier();  // ready: tile t+1 landed for every wave
            ml.read_frags(sa, sb, 0, fa[0], fb[0]);
            ML::mma(acc, fa[(KK - 1) & 1], fb[(KK - 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // ---- output epilogue: nothing is in flight any more
    epi(ml, acc);
}

// The loop variants an operation has, and the one every build includes.  Each
// variant is its own kernel: the host picks the one a call needs (a unit
// stride and small filter give masks, channel counts that are multiples of the
// K tile give whole taps per tile, K % 8 decides the ragged GEMM loop), so no
// loop carries a branch between its MFMAs and each loop gets its own register
// allocation (loops compiled into one kernel share one, and the largest ring's
// loops then spill).
template <class C, int V>
constexpr bool variant_applies() {
    if constexpr (C::GATHER_A) return V == PLAIN || V == UNIFORM_TAP || V == CONV_GENERIC;
    else if constexpr (C::WGRAD) return V == PLAIN;
    else return V == PLAIN || V == RAGGED;
}
template <class C>
constexpr int main_variant() { return C::GATHER_A ? UNIFORM_TAP : PLAIN; }

// End (exclusive) of stream-K workgroup g's run of K units.
__device__ __forceinline__ int64_t sk_end(int64_t total, int G, int g) { return total * (g + 1) / G; }

// One piece of work for a workgroup: the K range [kbase, kend) of output tile
// (tm, tn), and what to do with the accumulators afterwards.
enum Role : int {
    ROLE_STORE = 0,    // the whole K range: store the tile to C
    ROLE_SPLIT = 1,    // one split of a K split: store the fp32 partial tile to the workspace
    ROLE_PUBLISH = 2,  // a stream-K segment below the tile's last K unit: publish the partial
    ROLE_OWN = 3       // the stream-K segment with the tile's last K unit: collect, then store to C
};
struct WorkItem {
    int tm, tn, role, split;
    int64_t kbase, kend;
    int64_t tile_start;  // ROLE_OWN: the tile's first K unit in the concatenated stream-K range
};

// The stream-K workgroup's schedule, one item at a time.  Workgroup g first
// computes whole tiles g, g+G, ... below sk_dp_tiles (data-parallel rounds in
// the XCD order of tile_coords), then takes the K units [b, e) of the
// remaining tiles' concatenated K ranges and walks them backwards, one tile
// segment at a time, so that it first finishes the segment it shares with
// higher workgroups (publishing a partial) and last the segment whose tile it
// owns (collecting the partials of lower workgroups, which published theirs
// first).  An owner therefore only waits on workgroups dispatched no later
// than itself.
struct Schedule {
    int G, g;
    int64_t T, Tdp, UT, total, b, hi, blk;

    __device__ __forceinline__ explicit Schedule(const Params& p) {
        G = p.sk_grid;
        g = (int)blockIdx.x;
        T = (int64_t)p.tiles_m * p.tiles_n;
        Tdp = p.sk_dp_tiles;
        UT = p.sk_units;
        total = (T - Tdp) * UT;
        b = total * g / G;
        hi = sk_end(total, G, g);
        blk = g;
    }

    template <int UNIT>
    __device__ __forceinline__ bool next(const Params& p, WorkItem& it) {
        if (blk < Tdp) {
            tile_coords((int)blk, p.tiles_m, p.tiles_n, p.group_m, it.tm, it.tn);
            it.kbase = 0;
            it.kend = p.K;
            it.role = ROLE_STORE;
            it.split = 0;
            it.tile_start = 0;
            blk += G;
            return true;
        }
        if (hi <= b) return false;
        const int64_t tau = (hi - 1) / UT;
        const int64_t lo = b > tau * UT ? b : tau * UT;
        const int64_t u0 = lo - tau * UT, u1 = hi - tau * UT;
        // When every run holds whole tiles (c of them), the j-th tile of every
        // run is processed at the same time: give it the tile the
        // data-parallel grid runs in round j on the same XCD, keeping that
        // grid's L2 grouping.
        const int64_t Tsk = T - Tdp;
        int64_t block = tau;
        if (Tsk % G == 0 && (total / G) % UT == 0) {
            const int64_t c = Tsk / G;
            block = (tau % c) * G + tau / c;
        }
        tile_coords((int)(Tdp + block), p.tiles_m, p.tiles_n, p.group_m, it.tm, it.tn);
        it.kbase = u0 * UNIT;
        it.kend = u1 * UNIT < p.K ? u1 * UNIT : p.K;
        it.role = u1 < UT ? ROLE_PUBLISH : ROLE_OWN;
        it.split = 0;
        it.tile_start = tau * UT;
        hi = lo;
        return true;
    }
};

// After the K loop of one work item.  Every wave calls it.
template <class C, class ML>
__device__ __forceinline__ void finish_item(ML& ml, typename C::Acc (&acc)[C::FM][C::FN], const Params& p,
                                            const WorkItem& it, const Schedule& sch) {
    if (it.role == ROLE_STORE) {
        store_tile<C>(ml, acc, p.C, p.ldc, p.out_kind, p.vec_ok);
    } else if (it.role == ROLE_SPLIT) {
        ml.store(acc, p.ws + it.split * p.ws_stride, p.ldws, OUT_F32, true);
    } else if (it.role == ROLE_PUBLISH) {
        ml.sk_publish(acc, p.sk_ws + (int64_t)sch.g * (C::BM * C::BN), p.sk_flags + sch.g, sch.g != p.sk_drop);
    } else {
        // owner: add the partials of the lower workgroups sharing this tile, in
        // descending order; the wait for each is bounded, and a partial that
        // never arrives marks the tile (NaN) and the error word instead of
        // leaving a silently wrong result
        bool ok = true;
        for (int gp = sch.g - 1; gp >= 0 && sk_end(sch.total, sch.G, gp) > it.tile_start; --gp)
            ok = ml.sk_collect(acc, p.sk_ws + (int64_t)gp * (C::BM * C::BN), p.sk_flags + gp, p.sk_spin_limit,
                               (IGC_LDS int*)slot<C, 0>()) && ok;
        if (!ok) {
            constexpr int NE = (int)(sizeof(typename C::Acc) / sizeof(float));
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
#pragma unroll
                    for (int e = 0; e < NE; ++e) acc[i][j][e] = __builtin_nanf("");
            if (threadIdx.x == 0) __builtin_amdgcn_raw_buffer_store_b32(1, make_rsrc(p.err_word), 0, 0, 1 | 16);
        }
        store_tile<C>(ml, acc, p.C, p.ldc, p.out_kind, p.vec_ok);
    }
}

// The data-parallel kernel of loop variant V: one workgroup per output tile
// and K split.  It keeps no schedule state across its K loop: the loops of
// the largest tiles sit at the register limit, and any state kept alive around
// them spills inside.
template <class C, int V>
__global__ __launch_bounds__(C::NT) void gemm_kernel(const Params p) {
    static_assert(variant_applies<C, V>(), "loop variant of another operation");
    // work id = split * T + tile, in XCD order over the whole grid: with a K
    // split every XCD takes whole splits (or contiguous runs of one split's
    // tiles), so the A and B slices of a split are fetched into one L2 only
    const int T = p.tiles_m * p.tiles_n;
    const int id = xcd_order((int)blockIdx.x, T * p.k_splits);
    const int split = id / T;
    int tm, tn;
    group_coords(id - split * T, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int64_t kbase = (int64_t)split * p.k_per_split;
    const int64_t kend = kbase + p.k_per_split < p.K ? kbase + p.k_per_split : p.K;
    run_tile<C, V>(p, tm, tn, kbase, kend, [&](auto& ml, auto& acc) __attribute__((always_inline)) {
        if (p.k_splits > 1)
            ml.store(acc, p.ws + split * p.ws_stride, p.ldws, OUT_F32, true);
        else
            store_tile<C>(ml, acc, p.C, p.ldc, p.out_kind, p.vec_ok);
    });
}

// The stream-K kernel of loop variant V: the workgroup's work items one after
// another.
template <class C, int V>
__global__ __launch_bounds__(C::NT) void gemm_sk_kernel(const Params p) {
    static_assert(variant_applies<C, V>(), "loop variant of another operation");
    constexpr int UNIT = C::P * C::BK;  // stream-K unit: K elements of one ring period
    Schedule sch(p);
    WorkItem it;
    while (sch.template next<UNIT>(p, it)) {
        run_tile<C, V>(p, it.tm, it.tn, it.kbase, it.kend, [&](auto& ml, auto& acc) __attribute__((always_inline)) {
            finish_item<C>(ml, acc, p, it, sch);
        });
        __syncthreads();  // every wave is past this item's LDS before the next prologue
    }
}

}  // namespace igc
