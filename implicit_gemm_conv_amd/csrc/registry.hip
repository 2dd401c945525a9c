// registry.hip -- looks up compiled instances and picks the default tile.
#include "instances.hpp"

namespace igc {

static const igc_tune_t kTunes[] = {
#define IGC_TUNE_ENTRY(BM, BN, BK, D, W, MI, H, L, SY, F) {BM, BN, BK, D, W, MI, H, L == 0 ? W : L, 0, 0, SY, 0},
    IGC_FOR_EACH_TILE(IGC_TUNE_ENTRY)
#undef IGC_TUNE_ENTRY
};
static const int kScope[] = {
#define IGC_SCOPE_ENTRY(BM, BN, BK, D, W, MI, H, L, SY, F) F,
    IGC_FOR_EACH_TILE(IGC_SCOPE_ENTRY)
#undef IGC_SCOPE_ENTRY
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

int tune_scope(int i) { return kScope[i]; }

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
    // 256 x 256 output tiles, 8 waves, 16x16x32 MFMAs, loads issued by one
    // wave per SIMD.  The GEMM and the forward convolution use 64-deep K tiles
    // in a ring of two and a half stages (160 KB); the data gradient, whose
    // gathered A and row-major filter rows need more per-lane load state, uses
    // 32-deep K tiles in four stages (the 64-deep ring's loading waves spill).
    const igc_tune_t big = op == IGC_OP_CONV_DGRAD ? igc_tune_t{256, 256, 32, 4, 8, 16, 0, 4, 1, 0, 0, 0}
                                          : igc_tune_t{256, 256, 64, 2, 8, 16, 1, 4, 1, 0, 0, 0};
    // 128 x 128 tiles, 8 waves, 16x16x32 MFMAs, 64-deep K tiles in four stages.
    igc_tune_t small = {128, 128, 64, 4, 8, 16, 0, 4, 1, 0, 0, 0};
    // Whole rounds of tiles over the CUs decide: a round of 128 x 128 tiles
    // took 0.31 of a round of 256 x 256 tiles on the measured workloads (a
    // quarter of the work, at lower efficiency), so the larger tile wins unless
    // it leaves most of its last round idle or pads the output heavily.
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t r256 = (t256 + kCUs - 1) / kCUs, r128 = (t128 + kCUs - 1) / kCUs;
    if (t256 > 0 && r256 * 100 <= r128 * 31) {
        // A forward convolution whose 256-row tiles leave a last round partly idle may fill its rounds
        // better with 224-row tiles (7/8 of the work each): the 3x3 workload's 100,352 output pixels
        // make 392 tiles of 256 (1.53 rounds over 256 CUs) but 448 of 224 (1.75 rounds of 7/8 the
        // work).  Taken when whole rounds times rows per tile is smaller, and only where it is built.
        if (op == IGC_OP_CONV_FPROP) {
            const igc_tune_t b224 = {224, 256, 64, 2, 8, 16, 1, 4, 1, 0, 0, 0};
            const int64_t t224 = ((M + 223) / 224) * ((N + 255) / 256), r224 = (t224 + kCUs - 1) / kCUs;
            const Instance* e = find_instance(b224, false, true, true, IGC_OP_CONV_FPROP);
            if (e && e->full && r224 * 224 < r256 * 256) return b224;
        }
        return big;
    }
    // A forward convolution with a shallow K (a 1x1 filter, or few channels)
    // is bound by load latency rather than by the MFMAs: 64-column tiles in a
    // two-stage ring take 48 KB (128 rows, 4 waves) or 80 KB (256 rows, 8
    // waves) of LDS, so three or two workgroups share a CU and keep more loads
    // in flight.  Measured: the 1x1 workload (K = 64 outputs, C = 256) 38 ->
    // 19 us with 256 rows (20 us with 128), the C = 96, K = 192 3x3 workload
    // 30 -> 24 us with 128 rows (25 us with 256); a deep K (the 27 x 27 3x3
    // workload, C = 256) is slower with them (32-34 us against 25).
    if (op == IGC_OP_CONV_FPROP && K <= 1024 && N <= 256) {
        const igc_tune_t narrow = N <= 64 ? igc_tune_t{256, 64, 64, 2, 8, 16, 0, 4, 1, 0, 0, 0}
                                          : igc_tune_t{128, 64, 64, 2, 4, 16, 0, 0, 1, 0, 0, 0};
        const Instance* e = find_instance(narrow, false, true, true, IGC_OP_CONV_FPROP);
        if (e && e->full) return narrow;
    }
    // Small tiles.  When even they leave CUs idle and K is deep (at least 2048
    // per workgroup), the K work is spread over every CU.  An even K split
    // into S = CUs / tiles parts is taken when it fills at least 7/8 of the
    // CUs (each workgroup one part of a tile, the fp32 partials summed in
    // split order by the reduction kernel): it beats stream-K, whose runs
    // cross tile boundaries and make owners wait on other workgroups
    // (measured: 2048 x 1024 x 16384 2-way 75-80 us vs stream-K 82-87; the
    // filter gradient of the 3x3 workload, 36 tiles, 7-way 154-157 us vs
    // 182-185; 1000 x 1000 x 65536 4-way 167-171 vs 178-180).  Otherwise
    // stream-K over every CU.
    if (t128 > 0 && t128 < kCUs && K / 2048 >= 2) {
        // 256 x 128 tiles (three stages, wave sub-tiles of 128 x 32 against 64 x 32 for 128 x 128 tiles:
        // fewer LDS bytes per flop) split S ways, when that fills at least 7/8 of the CUs and leaves each
        // part 8192 or more of K.  Measured on 1000 x 1000 x 65536: 8 parts 151-163 us, against 158-185
        // for 16 parts of 256 x 256 tiles and 167-173 for 4 parts of 128 x 128; with 4096 per part
        // (2048 x 1024 x 16384: 4 parts) it only ties the 128 x 128 2-way split while doubling the partial
        // sums.  The filter gradient, whose operands both take transposing LDS reads, gains more and takes
        // it down to 2048 per part (the 3x3 workload's 18 tiles: 14 parts, 130-141 us against 154-192 for
        // 7 parts of 128 x 128).
        {
            igc_tune_t r = {256, 128, 64, 3, 8, 16, 0, 4, 1, 0, 0, 0};
            const int64_t tr = ((M + 255) / 256) * ((N + 127) / 128), sr = tr > 0 ? kCUs / tr : 0;
            const int64_t kmin = op == IGC_OP_CONV_WGRAD ? 2048 : 8192;
            const bool a_kc = op != IGC_OP_CONV_WGRAD, b_kc = op == IGC_OP_CONV_FPROP;
            const Instance* e = find_instance(r, false, a_kc, b_kc, op);
            if (e && e->full && sr >= 2 && sr * tr * 8 >= kCUs * 7 && K / sr >= kmin) {
                r.k_splits = (int)sr;
                return r;
            }
        }
        const int64_t s128 = kCUs / t128;
        if (s128 >= 2 && s128 * t128 * 8 >= kCUs * 7 && K / s128 >= 2048)
            small.k_splits = (int)s128;
        else
            small.stream_k = (int)kCUs;
    }
    return small;
}

}  // namespace igc
