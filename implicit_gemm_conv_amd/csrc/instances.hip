// instances.hip -- instantiates the mainloop kernel for one tile configuration
// (IGC_BM, IGC_BN, IGC_BK, IGC_D, IGC_W, IGC_MI, IGC_HALF, IGC_LW, IGC_SYNC
// given on the command line) and one operation family IGC_FAMILY:
//   0: bf16 GEMM (every operand layout; with IGC_FULL 0 only row-major A)
//   1: fp16 GEMM (every operand layout; with IGC_FULL 0 only row-major A)
//   2: forward convolution (bf16 and fp16; with IGC_FULL 0 bf16 only)
//   3: data gradient (bf16 and fp16)
//   4: filter gradient (bf16 and fp16)
// and registers the table when the library is loaded.  Every loop variant of
// an instance is a kernel of its own; IGC_SK 1 also builds the stream-K
// kernels.  With IGC_FULL 0 only the main loop variant is built (K % 8 == 0
// for the GEMM, whole filter taps per K tile and filters of at most 16 x 16
// for the convolution).
#include "instances.hpp"
#include "mainloop.hpp"

#if !defined(IGC_BM) || !defined(IGC_BN) || !defined(IGC_BK) || !defined(IGC_D) || !defined(IGC_W) || \
    !defined(IGC_MI) || !defined(IGC_HALF) || !defined(IGC_LW) || !defined(IGC_SYNC) || !defined(IGC_FULL) || \
    !defined(IGC_SK) || !defined(IGC_FAMILY)
#error "compile with -DIGC_BM=.. -DIGC_BN=.. -DIGC_BK=.. -DIGC_D=.. -DIGC_W=.. -DIGC_MI=.. -DIGC_HALF=.. -DIGC_LW=.. -DIGC_SYNC=.. -DIGC_FULL=.. -DIGC_SK=.. -DIGC_FAMILY=.."
#endif

namespace igc {

template <bool FP16, bool AKC, bool BKC, int OPK>
using Here = Cfg<FP16, IGC_BM, IGC_BN, IGC_BK, IGC_D, IGC_W, IGC_MI, IGC_HALF, IGC_LW, IGC_SYNC, AKC, BKC, OPK>;

// The kernel of loop variant V (stream-K when SK), or nullptr when the
// operation has no such variant or this build leaves it out.
template <class C, int V, bool SK>
constexpr const void* kernel_of() {
    if constexpr (!variant_applies<C, V>() || (!IGC_FULL && V != main_variant<C>()) || (SK && !IGC_SK))
        return nullptr;
    else if constexpr (SK)
        return reinterpret_cast<const void*>(&gemm_sk_kernel<C, V>);
    else
        return reinterpret_cast<const void*>(&gemm_kernel<C, V>);
}

template <bool FP16, bool AKC, bool BKC, int OPK>
Instance entry() {
    using C = Here<FP16, AKC, BKC, OPK>;
    return Instance{IGC_BM, IGC_BN, IGC_BK, IGC_D, IGC_W, IGC_MI, IGC_HALF, C::NL, IGC_SYNC, OPK, FP16, AKC, BKC,
                    IGC_FULL != 0,
                    {kernel_of<C, PLAIN, false>(), kernel_of<C, UNIFORM_TAP, false>(), kernel_of<C, RAGGED, false>(),
                     kernel_of<C, CONV_GENERIC, false>()},
                    {kernel_of<C, PLAIN, true>(), kernel_of<C, UNIFORM_TAP, true>(), kernel_of<C, RAGGED, true>(),
                     kernel_of<C, CONV_GENERIC, true>()},
                    C::LDS_BYTES};
}

#define IGC_ENTRY(FP16, AKC, BKC, OPK) entry<FP16, AKC, BKC, OPK>()

static const Instance kTable[] = {
#if IGC_FAMILY == 0
    IGC_ENTRY(false, true, true, OP_GEMM), IGC_ENTRY(false, true, false, OP_GEMM),
#if IGC_FULL
    IGC_ENTRY(false, false, true, OP_GEMM), IGC_ENTRY(false, false, false, OP_GEMM),
#endif
#elif IGC_FAMILY == 1
    IGC_ENTRY(true, true, true, OP_GEMM), IGC_ENTRY(true, true, false, OP_GEMM),
#if IGC_FULL
    IGC_ENTRY(true, false, true, OP_GEMM), IGC_ENTRY(true, false, false, OP_GEMM),
#endif
#elif IGC_FAMILY == 2
    IGC_ENTRY(false, true, true, OP_FPROP),
#if IGC_FULL
    IGC_ENTRY(true, true, true, OP_FPROP),
#endif
#elif IGC_FAMILY == 3
    IGC_ENTRY(false, true, false, OP_DGRAD), IGC_ENTRY(true, true, false, OP_DGRAD),
#elif IGC_FAMILY == 4
    IGC_ENTRY(false, false, false, OP_WGRAD), IGC_ENTRY(true, false, false, OP_WGRAD),
#else
#error "IGC_FAMILY must be 0..4"
#endif
};

namespace {
struct Registrar {
    Registrar() { register_instances(kTable, (int)(sizeof(kTable) / sizeof(kTable[0]))); }
};
const Registrar registrar;
}  // namespace

}  // namespace igc
