// registry.hip -- looks up compiled instances and picks the default tile.
#include "instances.hpp"

namespace igc {

static const igc_tune_t kTunes[] = {
#define IGC_TUNE_ENTRY(BM, BN, BK, D, W, MI, H, L) {BM, BN, BK, D, W, MI, H, L == 0 ? W : L, 0, 0},
    IGC_FOR_EACH_TILE(IGC_TUNE_ENTRY)
#undef IGC_TUNE_ENTRY
};

typedef const Instance* (*TableFn)(int*);
static const TableFn kTables[] = {
#define IGC_TABLE_ENTRY(BM, BN, BK, D, W, MI, H, L) &instance_table_##BM##x##BN##x##BK##x##D##x##W##x##MI##x##H##x##L,
    IGC_FOR_EACH_TILE(IGC_TABLE_ENTRY)
#undef IGC_TABLE_ENTRY
};

int num_tunes() { return (int)(sizeof(kTunes) / sizeof(kTunes[0])); }

igc_tune_t tune_at(int i) { return kTunes[i]; }

const Instance* find_instance(const igc_tune_t& q, bool fp16, bool a_kc, bool b_kc, bool conv) {
    const int mfma = q.mfma == 0 ? 32 : q.mfma;
    for (TableFn fn : kTables) {
        int n = 0;
        const Instance* t = fn(&n);
        for (int i = 0; i < n; ++i) {
            const Instance& e = t[i];
            if (e.bm == q.bm && e.bn == q.bn && e.bk == q.bk && e.d == q.pipe_depth && e.waves == q.waves &&
                e.mfma == mfma && e.half == q.half_stage && e.loaders == (q.loader_waves == 0 ? q.waves : q.loader_waves) &&
                e.fp16 == fp16 && e.a_kc == a_kc && e.b_kc == b_kc && e.conv == conv)
                return &e;
        }
    }
    return nullptr;
}

igc_tune_t default_tune(int64_t M, int64_t N, int64_t K, bool conv) {
    (void)conv;  // the GEMM and the convolution view take the same choice
    constexpr int64_t kCUs = 256;
    // Enough 256x256 tiles for every CU: the largest tile (least global and LDS
    // traffic per flop), 8 waves, 32-deep K tiles in a 4-stage ring, 16x16x32
    // MFMAs (which hold a higher clock than 32x32x16 under load) and loads
    // issued by one wave per SIMD: measured fastest, by a small margin, for
    // both the GEMM and the convolution once the output tile is stored
    // through LDS.
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    // 256x256 tiles unless they pad the output by more than a third more than
    // 128x128 tiles do (a 64-wide N, say) while 128x128 still fills the CUs
    const bool wasteful = t256 * 65536 * 3 > t128 * 16384 * 4 && t128 >= kCUs;
    if (t256 >= kCUs && !wasteful)
        return igc_tune_t{256, 256, 32, 4, 8, 16, 0, 4, 1, 0};
    // Otherwise 128x128 tiles; when even those leave CUs idle and K is deep
    // (at least 2048 per CU's share), stream-K over every CU balances the K
    // work; shallow K runs one tile per workgroup.
    if (t128 > 0 && t128 < kCUs && K / 2048 >= 2)
        return igc_tune_t{128, 128, 64, 4, 4, 32, 0, 4, 1, (int)kCUs};
    return igc_tune_t{128, 128, 64, 4, 4, 32, 0, 4, 1, 0};
}

}  // namespace igc
