// registry.hip -- looks up compiled instances and picks the default tile.
#include "instances.hpp"

namespace igc {

static const igc_tune_t kTunes[] = {
#define IGC_TUNE_ENTRY(BM, BN, BK, D, W, MI, H, L, SY, F) {BM, BN, BK, D, W, MI, H, L == 0 ? W : L, 0, 0, SY, 0},
    IGC_FOR_EACH_TILE(IGC_TUNE_ENTRY)
#undef IGC_TUNE_ENTRY
};
static const bool kFull[] = {
#define IGC_FULL_ENTRY(BM, BN, BK, D, W, MI, H, L, SY, F) F != 0,
    IGC_FOR_EACH_TILE(IGC_FULL_ENTRY)
#undef IGC_FULL_ENTRY
};

// Tables registered by the instance objects while the library loads (static
// initialisers run one at a time, before any entry point can be called).
constexpr int kMaxTables = 256;
static const Instance* g_tables[kMaxTables];
static int g_counts[kMaxTables];
static int g_ntables = 0;

void register_instances(const Instance* table, int count) {
    if (g_ntables < kMaxTables) {
        g_tables[g_ntables] = table;
        g_counts[g_ntables] = count;
        ++g_ntables;
    }
}

int num_tunes() { return (int)(sizeof(kTunes) / sizeof(kTunes[0])); }

igc_tune_t tune_at(int i) { return kTunes[i]; }

bool tune_is_full(int i) { return kFull[i]; }

const Instance* find_instance(const igc_tune_t& q, bool fp16, bool a_kc, bool b_kc, int op) {
    const int mfma = q.mfma == 0 ? 32 : q.mfma;
    const int loaders = q.loader_waves == 0 ? q.waves : q.loader_waves;
    for (int t = 0; t < g_ntables; ++t) {
        for (int i = 0; i < g_counts[t]; ++i) {
            const Instance& e = g_tables[t][i];
            if (e.bm == q.bm && e.bn == q.bn && e.bk == q.bk && e.d == q.pipe_depth && e.waves == q.waves &&
                e.mfma == mfma && e.half == q.half_stage && e.loaders == loaders && e.sync == q.ring_sync &&
                e.fp16 == fp16 && e.a_kc == a_kc && e.b_kc == b_kc && e.op == op)
                return &e;
        }
    }
    return nullptr;
}

igc_tune_t default_tune(int64_t M, int64_t N, int64_t K, int op) {
    constexpr int64_t kCUs = 256;
    igc_tune_t t = {256, 256, 32, 4, 8, 16, 0, 4, 1, 0, 0, 0};
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
    if (t256 >= kCUs && !wasteful) {
        // A last round of tiles that leaves CUs idle (for the 3x3 convolution,
        // 392 tiles = 1.53 rounds) is spread over every CU: whole tiles in
        // data-parallel rounds, then the remaining tiles' K ranges cut into
        // equal runs (stream-K), when the K range is deep enough to split.
        const int64_t rem = t256 % kCUs;
        if (rem != 0 && rem * 4 < kCUs * 3 && K >= 1024) {
            t.stream_k = (int)kCUs;
            t.sk_hybrid = 1;
        }
        (void)op;
        return t;
    }
    // Otherwise 128x128 tiles; when even those leave CUs idle and K is deep
    // (at least 2048 per CU's share), stream-K over every CU balances the K
    // work; shallow K runs one tile per workgroup.
    t = igc_tune_t{128, 128, 64, 4, 4, 32, 0, 4, 1, 0, 0, 0};
    if (t128 > 0 && t128 < kCUs && K / 2048 >= 2) t.stream_k = (int)kCUs;
    return t;
}

}  // namespace igc
