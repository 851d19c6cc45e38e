// plan_sweep.cpp -- sweeps libnmspmv's launch planners (nm_plan.h) and argument
// rules (nm_rules.h) over matrix shapes, batches, CU counts and the tuning
// overrides, and checks every plan against what the kernels assume of it:
// block size, LDS within the CU's 160 KB, rows and chunks fully covered, x
// staging that fits.  The CPU tests build it with -fsanitize=address,undefined
// (any undefined behaviour or bad access aborts the run); a violated
// invariant prints the case and exits 1.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <set>
#include <utility>
#include <vector>

#include "nm_plan.h"

using namespace nmh;

namespace {

int g_cus = 256;
long g_plans = 0;
long g_kinds[8] = {};   // plans seen per kernel kind (0: fused hybrid, 2: K-split ring)
char g_case[256];

#define REQUIRE(c)                                                                         \
    do {                                                                                   \
        if (!(c)) {                                                                        \
            std::fprintf(stderr, "violated: %s  [%s]  line %d\n", #c, g_case, __LINE__);   \
            std::exit(1);                                                                  \
        }                                                                                  \
    } while (0)

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// The row-slice kernel's slice length in chunks (rounded to 32) for C chunks over S slices.
int64_t slice_chunks(int64_t C, int S, int ls) { return (((C + S - 1) >> ls) + 31) & ~int64_t(31); }

template <int F>
void check_rowslice(const Plan& P, int64_t R, int64_t K, int B, bool glu)
{
    const int64_t C = K / chunk_cols<F>();
    const size_t xbytes = (size_t)B * (size_t)x_row_units(K) * 16;
    REQUIRE(pow2(P.S) && P.S <= 16 && (1 << P.ls) == P.S);
    REQUIRE(P.rpw == 1 || P.rpw == 2);
    const int waves = P.rpb / P.rpw;            // rpb counts rows: rpw a wave
    REQUIRE(P.rpb % P.rpw == 0 && waves >= 1 && waves * P.S <= 16 && P.threads == waves * P.S * kWave);
    if (P.rpw == 2)                             // the instantiated row-pair kernels
        REQUIRE(F != kDense && P.S == 1 && B >= 1 && B <= 4 && (P.cpl == 4 || P.cpl == 5) &&
                (B >= 3 || g_env.rpw == 2) && rowslice_x_regs(B, K, P.threads, P.cpl) <= 1);
    REQUIRE(P.cpl >= 1 && P.cpl <= (B == 1 && !glu && F != kDense ? 16 : 8));
    REQUIRE(slice_chunks(C, P.S, P.ls) <= 64LL * P.cpl);
    REQUIRE((int64_t)P.grid * P.rpb >= R && ((int64_t)P.grid - 1) * P.rpb < R);
    REQUIRE(xbytes <= (size_t)kXTileBudget);
    REQUIRE(P.lds >= (size_t)table_units<F>() * kUnitBytes + xbytes + (size_t)P.rpb * P.S * B * 4);
    if (glu)
        REQUIRE(P.rpb % 2 == 0);
    const int xu = rowslice_x_regs(B, K, P.threads, P.cpl);
    REQUIRE(xu == 0 || xu == 1 || (xu == 4 && B == 1 && P.cpl <= 8));
    if (xu != 0)
        REQUIRE((int64_t)xu * P.threads >= (int64_t)B * (K / 8));
}

template <int F>
void check_valu(int64_t R, int64_t K, int B, bool glu)
{
    const Plan P = plan_for<F>(R, K, B, glu);
    ++g_plans;
    ++g_kinds[P.kind & 7];
    REQUIRE(P.lds <= (size_t)kLdsMax);
    REQUIRE(P.threads % kWave == 0 && P.threads >= kWave && P.threads <= 1024);
    REQUIRE(P.grid >= 1);
    if (P.kind == 1) {
        check_rowslice<F>(P, R, K, B, glu);
    } else {
        REQUIRE(P.kind == 3);
        REQUIRE(P.tile_cols == K || (P.tile_cols > 0 && P.tile_cols % 1024 == 0 && P.tile_cols < K));
        const int nw = P.threads / kWave, per = glu ? 2 : 1;
        const int64_t G = (int64_t)P.grid * nw, Ru = R / per;
        size_t need = (size_t)table_units<F>() * kUnitBytes + (size_t)B * x_row_units(P.tile_cols) * 16;
        if (P.tile_cols < K)                     // the kernel's per-wave partial sums across x tiles
            need += (size_t)nw * (size_t)(per * ((Ru + G - 1) / G)) * B * 4;
        REQUIRE(P.lds >= need);
    }
    if (F != kDense && !glu && B <= 3) {
        Plan H;
        if (plan_hybrid<F>(R, K, B, &H)) {
            ++g_plans;
            ++g_kinds[0];
            REQUIRE(H.kind == 1 && H.rpb >= 2 && H.rpb % 2 == 0 && H.rpw == 1);
            check_rowslice<F>(H, R, K, B, false);
            REQUIRE(H.lds <= (size_t)kLdsMax);
            // the dense rows: half the rows per block over twice the slices, K / 8 chunks a row
            REQUIRE(slice_chunks(K / 8, 2 * H.S, H.ls + 1) <= 64LL * H.cpl);
        }
    }
}

// LDS the shared-x ring kernel addresses: the selector table, then per wave
// two slots of TW tiles (values, and masks for sparse rows), then the
// block's two x slots of the batch rows (padded to whole load instructions)
// times one stage of x.
template <int F>
size_t shared_ring_lds(int waves, int TW, int B)
{
    const size_t tile = kRingValues + (F == kDense ? 0 : kRingMasks);
    const size_t x = (size_t)ring_x_rows<F>(B) * ring_x_units<F>() * 16;
    return (size_t)mfma_table_units<F>() * kUnitBytes + (size_t)waves * 2 * TW * tile + 2 * x;
}

template <int F>
void check_mfma(int64_t R, int64_t K, int B, bool glu)
{
    const int64_t tiles16 = (R + 15) / 16;
    if (mfma_use_ring<F>(R, K, B)) {
        REQUIRE(F == kDense || K % 32 == 0);
        const Plan P = plan_mfma_ring<F>(R, K, B);
        ++g_plans;
        ++g_kinds[P.kind & 7];
        const int TW = P.cpl;
        REQUIRE(TW == 1 || TW == 2);
        if (B > 16)
            REQUIRE(TW == 2);
        REQUIRE(P.threads % kWave == 0 && P.threads >= kWave && P.threads <= 512);
        REQUIRE(P.lds <= (size_t)kLdsMax);
        const int64_t tiles = (R + 16 * TW - 1) / (16 * TW);
        if (P.kind == 6) {
            REQUIRE(P.threads == P.S * kWave && P.rpb == 1);
            REQUIRE((int64_t)P.grid == tiles);
        } else {
            REQUIRE(P.kind == 7 && P.S == 1 && P.threads == P.rpb * kWave);
            REQUIRE(P.lds >= shared_ring_lds<F>(P.rpb, TW, B));
            if (P.map_k == 0) {
                REQUIRE((int64_t)P.grid * P.rpb >= tiles && ((int64_t)P.grid - 1) * P.rpb < tiles);
            } else {
                // CU-major map, as the kernel computes it: every tile in exactly one
                // block, no block with more tiles than waves, one round of blocks
                REQUIRE(TW == 1 && P.map_cus == g_cus && P.map_k >= 1 && (int64_t)P.grid == (int64_t)P.map_k * g_cus);
                REQUIRE((int64_t)(kLdsMax / P.lds) >= P.map_k && P.map_k * P.rpb <= 20);
                std::vector<std::pair<int64_t, int64_t>> parts;
                for (int64_t b = 0; b < P.grid; ++b) {
                    const int64_t c = b % P.map_cus, j = b / P.map_cus;
                    const int64_t s0 = c * tiles / P.map_cus, n = (c + 1) * tiles / P.map_cus - s0;
                    const int64_t f = s0 + j * n / P.map_k, l = s0 + (j + 1) * n / P.map_k;
                    REQUIRE(f <= l && l - f <= P.rpb);
                    if (l > f)
                        parts.emplace_back(f, l);
                }
                std::sort(parts.begin(), parts.end());
                int64_t next = 0;
                for (const auto& pr : parts) {
                    REQUIRE(pr.first == next);
                    next = pr.second;
                }
                REQUIRE(next == tiles);
            }
        }
    } else {
        const int NT = B > 16 ? 2 : 1;
        const Plan P = plan_mfma_stage<F>(R, K, NT, B);
        ++g_plans;
        ++g_kinds[P.kind & 7];
        REQUIRE(P.kind == 5 && P.S >= 1 && P.S <= 8 && P.rpb >= 1);
        REQUIRE(P.threads == P.S * P.rpb * kWave && P.threads <= 512);
        REQUIRE(P.lds <= (size_t)kLdsMax);
        REQUIRE((int64_t)P.grid * P.rpb >= tiles16 && ((int64_t)P.grid - 1) * P.rpb < tiles16);
    }
    Plan SP;
    if (mfma_use_split<F>(R, K, B, &SP)) {
        REQUIRE(F == kDense || K % 32 == 0);
        ++g_plans;
        ++g_kinds[2];
        const int64_t NS = (K / chunk_cols<F>() + kStageChunks - 1) / kStageChunks;
        const int W = SP.rpb, TWs = SP.cpl, NTs = B > 16 ? 2 : 1;
        REQUIRE(SP.kind == 8 && SP.S == 1 && (TWs == 1 || TWs == 2) && (B <= 16 || TWs == 2));
        REQUIRE(W >= 1 && SP.threads == W * kWave && SP.threads <= 512);
        REQUIRE(SP.lds <= (size_t)kLdsMax && SP.lds >= shared_ring_lds<F>(W, TWs, B));
        REQUIRE(SP.ks >= 2 && SP.ks <= 32 && SP.kstages >= 1);
        REQUIRE((int64_t)SP.ks * SP.kstages >= NS);                      // every stage in some split
        const int64_t groups = SP.grid / SP.ks;
        REQUIRE((int64_t)SP.grid == groups * SP.ks && groups <= kSplitMaxGroups);
        REQUIRE(groups * W * 16 * TWs >= R);                               // every row in some tile
        REQUIRE((size_t)SP.ks * groups * W * TWs * NTs * 1024 <= kSplitPartBytes);
    }
    (void)glu;
}

template <int F>
void sweep_format(const char* env_name)
{
    static const int64_t Rs[] = {1, 2, 3, 7, 16, 17, 63, 64, 65, 1000, 1024, 4096, 5120, 14336, 25600, 28672,
                                 int64_t(1) << 20, kRowLimit - 2};
    static const int64_t Ks[] = {8, 16, 24, 32, 48, 64, 1008, 1024, 2048, 2064, 4096, 5120, 8192, 8200, 13824, 14336,
                                 16384, 18432, 18448, 25600, 28672, 32768, 65536, int64_t(1) << 20, 2147483632};
    static const int Bs[] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 17, 24, 32};
    for (int64_t R : Rs)
        for (int64_t K : Ks) {
            if (K % (F == kDense ? 8 : 16) != 0)
                continue;
            for (int B : Bs)
                for (int glu = 0; glu < 2; ++glu) {
                    const int64_t Rl = glu ? 2 * (R / 2 + 1) : R;   // gated launches interleave row pairs
                    if (Rl >= kRowLimit)
                        continue;
                    std::snprintf(g_case, sizeof g_case, "env %s, cus %d, fmt %d, R %lld, K %lld, B %d, glu %d",
                                  env_name, g_cus, F, (long long)Rl, (long long)K, B, glu);
                    const bool mfma = use_mfma<F>(Rl, K, B, glu != 0);
                    if (B > kVectorMaxBatch)
                        REQUIRE(mfma);
                    if (mfma)
                        check_mfma<F>(Rl, K, B, glu != 0);
                    else
                        check_valu<F>(Rl, K, B, glu != 0);
                }
        }
}

struct Override {
    const char* name;
    int Env::*field;
    int value;
};

void check_rules()
{
    std::snprintf(g_case, sizeof g_case, "argument rules");
    // overlaps against brute force over small address ranges (0 = no buffer)
    for (uintptr_t a = 0; a < 24; ++a)
        for (size_t na = 0; na < 6; ++na)
            for (uintptr_t b = 0; b < 24; ++b)
                for (size_t nb = 0; nb < 6; ++nb) {
                    std::set<uintptr_t> sa;
                    bool any = false;
                    if (a != 0)
                        for (size_t i = 0; i < na; ++i)
                            sa.insert(a + i);
                    if (b != 0)
                        for (size_t i = 0; i < nb; ++i)
                            any = any || sa.count(b + i) != 0;
                    const bool got = overlaps(reinterpret_cast<const void*>(a), na, reinterpret_cast<const void*>(b), nb);
                    REQUIRE(got == any);
                    REQUIRE(got == overlaps(reinterpret_cast<const void*>(b), nb, reinterpret_cast<const void*>(a), na));
                }
    // pointer presence and alignment
    for (uintptr_t p = 0; p < 64; ++p)
        for (uintptr_t al : {1u, 2u, 4u, 8u, 16u})
            for (size_t n : {size_t(0), size_t(1), size_t(100)}) {
                const bool want = n == 0 || (p != 0 && p % al == 0);
                REQUIRE(ptr_ok(reinterpret_cast<const void*>(p), n, al) == want);
            }
    // shape limits, including the extremes of int64
    const int64_t vals[] = {INT64_MIN, -(int64_t(1) << 40), -16, -8, -1, 0, 1, 7, 8, 12, 16, 24, 4096,
                            INT32_MAX - 7, INT32_MAX, int64_t(INT32_MAX) + 1, kRowLimit - 1, kRowLimit,
                            int64_t(1) << 40, INT64_MAX - 7, INT64_MAX};
    for (int64_t R : vals)
        for (int64_t K : vals) {
            const bool want = R >= 0 && R < kRowLimit && K >= 0 && K <= INT32_MAX && K % 8 == 0;
            REQUIRE((check_rk(R, K) == NM_OK) == want);
            for (int M = -1; M <= 9; ++M)
                for (int N = -1; N <= 9; ++N) {
                    const bool ok = (M == 4 || M == 8) && N >= 1 && N < M && K % M == 0;
                    REQUIRE((check_nm(K, N, M) == NM_OK) == ok);
                }
        }
    for (int B = -2; B <= 40; ++B)
        REQUIRE((check_batch(B) == NM_OK) == (B >= 1 && B <= kMaxBatch));
    for (int d = -3; d <= 3; ++d)
        REQUIRE((check_dtype(d) == NM_OK) == (d == NM_FP16 || d == NM_BF16));
    for (int v = 1; v <= 1024; ++v) {
        const int l = log2_exact(v);
        REQUIRE((1 << l) <= v && v < (2 << l));
    }
}

}  // namespace

int nmh::cu_count() { return g_cus; }

int main()
{
    std::call_once(g_env_once, read_env);       // run with no NMSPMV_* variables set
    check_rules();
    const Env defaults = g_env;
    const Override overrides[] = {
        {"default", nullptr, 0},
        {"kernel=1", &Env::kernel, 1},          {"kernel=3", &Env::kernel, 3},
        {"kernel=5", &Env::kernel, 5},          {"kernel=6", &Env::kernel, 6},
        {"slices=1", &Env::slices, 1},          {"slices=4", &Env::slices, 4},
        {"slices=16", &Env::slices, 16},        {"slices=100", &Env::slices, 100},
        {"rpb=1", &Env::rpb, 1},                {"rpb=3", &Env::rpb, 3},
        {"rpb=16", &Env::rpb, 16},              {"threads=64", &Env::threads, 64},
        {"threads=1024", &Env::threads, 1024},  {"threads=100", &Env::threads, 100},
        {"tile_bytes=1", &Env::tile_bytes, 1},  {"tile_bytes=4096", &Env::tile_bytes, 4096},
        {"blocks=1", &Env::blocks, 1},          {"blocks=100000", &Env::blocks, 100000},
        {"mfma_min_b=2", &Env::mfma_min_b, 2},  {"mfma_slices=1", &Env::mfma_slices, 1},
        {"mfma_slices=3", &Env::mfma_slices, 3}, {"mfma_slices=8", &Env::mfma_slices, 8},
        {"ring_tiles=1", &Env::ring_tiles, 1},  {"ring_tiles=2", &Env::ring_tiles, 2},
        {"ring_share=1", &Env::ring_share, 1},  {"ring_share=8", &Env::ring_share, 8},
        {"xfirst=0", &Env::xfirst, 0},          {"xfirst=1", &Env::xfirst, 1},
        {"blocks_per_cu=2", &Env::blocks_per_cu, 2}, {"blocks_per_cu=8", &Env::blocks_per_cu, 8},
        {"xdma=1", &Env::xdma, 1},              {"max_cpl=14", &Env::max_cpl, 14},
        {"max_cpl=16", &Env::max_cpl, 16},      {"max_cpl=100", &Env::max_cpl, 100},
        {"splitk=1", &Env::splitk, 1},          {"splitk=2", &Env::splitk, 2},
        {"splitk_ks=3", &Env::splitk_ks, 3},    {"splitk_ks=32", &Env::splitk_ks, 32},
        {"rpw=1", &Env::rpw, 1},                {"rpw=2", &Env::rpw, 2},
    };
    for (int cus : {256, 80, 1}) {
        g_cus = cus;
        for (const Override& o : overrides) {
            g_env = defaults;
            if (o.field)
                g_env.*(o.field) = o.value;
            sweep_format<kDense>(o.name);
            sweep_format<kNM24>(o.name);
            sweep_format<kNM48>(o.name);
        }
    }
    std::printf("plan sweep: %ld plans checked (fused hybrid %ld, row-slice %ld, stream %ld, staged %ld, ring %ld, "
                "shared-x ring %ld, K-split ring %ld)\n", g_plans, g_kinds[0], g_kinds[1], g_kinds[3], g_kinds[5],
                g_kinds[6], g_kinds[7], g_kinds[2]);
    std::snprintf(g_case, sizeof g_case, "coverage");
    for (int k : {0, 1, 2, 3, 5, 6, 7})
        REQUIRE(g_kinds[k] > 0);            // every kernel's plan was reached
    return 0;
}
