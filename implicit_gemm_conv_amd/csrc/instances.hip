// instances.hip -- instantiates the mainloop kernel for one tile configuration
// (IGC_BM, IGC_BN, IGC_BK, IGC_D, IGC_W, IGC_MI, IGC_HALF, IGC_LW given on the command line) with
// every input type and operand layout: 8 GEMM kernels and 2 implicit-GEMM conv
// kernels.
#include "instances.hpp"
#include "mainloop.hpp"

#if !defined(IGC_BM) || !defined(IGC_BN) || !defined(IGC_BK) || !defined(IGC_D) || !defined(IGC_W) || \
    !defined(IGC_MI) || !defined(IGC_HALF) || !defined(IGC_LW)
#error "compile with -DIGC_BM=.. -DIGC_BN=.. -DIGC_BK=.. -DIGC_D=.. -DIGC_W=.. -DIGC_MI=.. -DIGC_HALF=.. -DIGC_LW=.."
#endif

#define IGC_CAT9(a, b, c, d, e, f, g, h, i) a##b##x##c##x##d##x##e##x##f##x##g##x##h##x##i
#define IGC_TABLE_NAME(BM, BN, BK, D, W, MI, H, L) IGC_CAT9(instance_table_, BM, BN, BK, D, W, MI, H, L)

namespace igc {

template <bool FP16, bool AKC, bool BKC, bool CONV>
using Here = Cfg<FP16, IGC_BM, IGC_BN, IGC_BK, IGC_D, IGC_W, IGC_MI, IGC_HALF, IGC_LW, AKC, BKC, CONV>;

#define IGC_ENTRY(FP16, AKC, BKC, CONV)                                                                   \
    Instance {                                                                                           \
        IGC_BM, IGC_BN, IGC_BK, IGC_D, IGC_W, IGC_MI, IGC_HALF, Here<FP16, AKC, BKC, CONV>::NL, FP16, AKC, BKC, \
            CONV,                                                                                        \
            reinterpret_cast<const void*>(&gemm_kernel<Here<FP16, AKC, BKC, CONV>>),                     \
            Here<FP16, AKC, BKC, CONV>::LDS_BYTES                                                        \
    }

static const Instance kTable[] = {
    IGC_ENTRY(false, true, true, false),  IGC_ENTRY(false, true, false, false),
    IGC_ENTRY(false, false, true, false), IGC_ENTRY(false, false, false, false),
    IGC_ENTRY(true, true, true, false),   IGC_ENTRY(true, true, false, false),
    IGC_ENTRY(true, false, true, false),  IGC_ENTRY(true, false, false, false),
    IGC_ENTRY(false, true, true, true),   IGC_ENTRY(true, true, true, true),
};

const Instance* IGC_TABLE_NAME(IGC_BM, IGC_BN, IGC_BK, IGC_D, IGC_W, IGC_MI, IGC_HALF, IGC_LW)(int* count) {
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace igc
