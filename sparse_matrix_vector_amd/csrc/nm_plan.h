// nm_plan.h -- libnmspmv's launch planning: the LDS layout constants the
// kernels and the planner share, and the rules that pick a kernel and its
// launch shape for a matrix shape and batch.
//
// Host-only C++ apart from the constexpr helpers (which the kernels also use):
// no HIP headers, so that a plain C++ compiler, with sanitizers, can sweep
// the planners without a GPU.  cu_count() is supplied by the library (the
// current device's compute units) or by such a test.
#ifndef NM_PLAN_H
#define NM_PLAN_H

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "nm_rules.h"

namespace nmh {

constexpr int kWave = 64;
constexpr int kXTileBudget = 56 * 1024;   // LDS bytes for x in the row-slice / stream kernels
constexpr int kXTileStream = 64 * 1024;   // LDS bytes per x tile in the stream kernel
constexpr int kLdsMax = 160 * 1024;       // LDS per CU on gfx950

enum Fmt { kDense = 0, kNM24 = 1, kNM48 = 2 };

// 16-byte units of the selector table each format keeps in LDS.
template <int F>
constexpr int table_units()
{
    return F == kNM24 ? 4 : (F == kNM48 ? 16 : 0);
}

template <int F>
constexpr int chunk_cols()
{
    return F == kDense ? 8 : 16;
}

constexpr int kUnitBytes = 16;            // one chunk, one x unit, one selector-table entry

// LDS units per batch row of x for K staged columns: K/8 rounded up to whole
// 64-unit runs.
constexpr int x_row_units(int64_t K)
{
    return (int)(((K / 8) + 63) / 64 * 64);
}

// 16-byte LDS units of the matrix-core kernels' expansion tables.  2:4: one
// expand24 selector pair per nibble (16 entries of 8 bytes: 64 lanes reading
// arbitrary entries touch distinct banks or share a word); 4:8: the VALU
// kernels' two 16-entry nibble tables of 8-byte entries.
template <int F>
constexpr int mfma_table_units()
{
    return F == kDense ? 0 : F == kNM24 ? 8 : 16;
}

// Staged matrix-core kernel: per wave, a 16-row tile's values and masks for
// one stage of 16 chunks per row, rows padded apart in LDS banks.
constexpr int kStageChunks = 16;                                  // chunks per row per stage
constexpr int kStagePitch = kStageChunks * 16 + 16;               // bytes per values row (rows 4 banks apart)
constexpr int kStageMPitch = kStageChunks * 2 + 8;                // bytes per mask row (8-byte reads, rows 10 banks apart)
constexpr int kStageBytes = 16 * kStagePitch + 16 * kStageMPitch; // per wave

// LDS-ring matrix-core kernel: one ring slot's values and masks of a 16-row tile.
constexpr int kRingValues = 16 * kStageChunks * 16;               // 4 KB
constexpr int kRingMasks = 16 * kStageChunks * 2;                 // 512 B

// x units (16 bytes) per batch row per stage.
template <int F>
constexpr int ring_x_units()
{
    return kStageChunks * chunk_cols<F>() / 8;
}

// Batch rows of x staged per slot: B rounded up to whole load instructions
// (64 lanes of 16 bytes).
template <int F>
constexpr int ring_x_rows(int B)
{
    return (B + kWave / ring_x_units<F>() - 1) / (kWave / ring_x_units<F>()) * (kWave / ring_x_units<F>());
}

// One ring slot: TW tiles' values and masks, then the stage's x.
template <int F, int TW>
constexpr int ring_slot_bytes(int B)
{
    return TW * (kRingValues + (F == kDense ? 0 : kRingMasks)) + ring_x_rows<F>(B) * ring_x_units<F>() * 16;
}

// Compute units of the current device (256 on MI355X).
int cu_count();

// ---- launch planning -------------------------------------------------------------

// Launch-shape overrides, read once, for tuning sweeps (0 = built-in choice):
// NMSPMV_KERNEL 1 = row-slice, 3 = stream, 5 = staged matrix-core (instead of
// the LDS ring), 6 = the LDS ring wherever K allows it; NMSPMV_SLICES, NMSPMV_ROWS_PER_BLOCK (row-slice);
// NMSPMV_BLOCKS, NMSPMV_THREADS, NMSPMV_TILE_BYTES (stream);
// NMSPMV_MFMA_MIN_B (smallest batch sent to the matrix-core kernels),
// NMSPMV_MFMA_SLICES; NMSPMV_HYBRID_SPLIT=1 runs a hybrid matrix's sparse and
// dense rows as two launches; NMSPMV_XFIRST=0/1 turns the row-slice kernel's
// x-first issue order off/on (default: on where a row is cut into slices);
// NMSPMV_BLOCKS_PER_CU (2 to 8) caps a row-slice launch's resident blocks
// per CU by padding its LDS; NMSPMV_XDMA=1 stages x by global-to-LDS loads
// wherever one register per thread does not cover it; NMSPMV_MAX_CPL (9 to
// 16) lets a single-vector sparse row of up to that many chunks per lane run
// on one wave instead of being cut into slices; NMSPMV_SPLITK=1 turns the
// K-split ring plan off, 2 uses it wherever it fits (with a workspace);
// NMSPMV_SPLITK_KS sets its split count (2 to 32); NMSPMV_RPW=1 turns the
// row-slice kernel's row pairs (two rows a wave) off, 2 takes them from one
// vector (default: 3 and 4).
struct Env {
    int kernel = 0, slices = 0, rpb = 0, blocks = 0, threads = 0, tile_bytes = 0, mfma_min_b = 0, mfma_slices = 0,
        ring_tiles = 0, ring_share = 0, hybrid_split = 0, xfirst = -1, blocks_per_cu = 0, xdma = 0, max_cpl = 0,
        splitk = 0, splitk_ks = 0, rpw = 0;
};
inline Env g_env;
inline std::once_flag g_env_once;

inline void read_env()
{
    auto get = [](const char* name) {
        const char* e = std::getenv(name);
        return e ? std::atoi(e) : 0;
    };
    g_env.kernel = get("NMSPMV_KERNEL");
    g_env.slices = get("NMSPMV_SLICES");
    g_env.rpb = get("NMSPMV_ROWS_PER_BLOCK");
    g_env.blocks = get("NMSPMV_BLOCKS");
    g_env.threads = get("NMSPMV_THREADS");
    g_env.tile_bytes = get("NMSPMV_TILE_BYTES");
    g_env.mfma_min_b = get("NMSPMV_MFMA_MIN_B");
    g_env.mfma_slices = get("NMSPMV_MFMA_SLICES");
    g_env.ring_tiles = get("NMSPMV_RING_TILES");
    g_env.ring_share = get("NMSPMV_RING_SHARE");
    g_env.hybrid_split = get("NMSPMV_HYBRID_SPLIT");
    g_env.blocks_per_cu = get("NMSPMV_BLOCKS_PER_CU");
    g_env.xdma = get("NMSPMV_XDMA");
    g_env.max_cpl = get("NMSPMV_MAX_CPL");
    g_env.splitk = get("NMSPMV_SPLITK");
    g_env.splitk_ks = get("NMSPMV_SPLITK_KS");
    g_env.rpw = get("NMSPMV_RPW");
    const char* xf = std::getenv("NMSPMV_XFIRST");
    g_env.xfirst = xf ? std::atoi(xf) : -1;
}

struct Plan {
    int kind = 0;            // 1 row-slice, 3 stream
    int S = 1, rpb = 1, cpl = 1, threads = 256, tile_cols = 0;
    int ls = 0;              // log2(S) (row-slice: S is a power of two)
    int rpw = 1;             // row-slice: rows a wave (2: row pairs; rpb counts rows)
    int xf = 0;              // row-slice: x loads issued by the whole block before any weight load
    int ks = 0, kstages = 0; // K-split ring (kind 8): splits, stages per split
    int map_k = 0, map_cus = 0; // shared-x ring (kind 7): CU-major tile map, k blocks a CU (0: plain)
    size_t lds = 0;
    unsigned grid = 1;
};

inline int log2_exact(int v)
{
    int l = 0;
    while ((1 << (l + 1)) <= v)
        ++l;
    return l;
}

// Row-slice shape (rules from timing sweeps on MI355X over the Llama-3.1-8B,
// Llama-3.3-70B and Qwen3 projection shapes, sparse and dense):
//  * sparse rows of <= 320 chunks: one wave per row, 8 rows per block;
//    longer: the fewest slices S >= 2 (a power of two) that keep a lane at
//    <= 8 chunks, 8 / S rows per block;
//  * dense rows of <= 512 chunks: one wave per row, 4 rows per block;
//    longer: the fewest slices that keep a lane at <= 7 chunks, 8 / S rows;
//  * few rows (under ~16 waves per CU): more slices, down to 64 chunks each;
//  * at least two blocks per CU;
//  * blocks of at most 8 waves: 16-wave blocks (tried for the Llama-3.1-8B
//    down projection, 4096 x 14336) timed 12.5 us on some MI355X GPUs and
//    13.7-14.9 us, with a wide spread between launches, on others, where
//    8-wave blocks held 12.4-12.5 us on all of them;
//  * rows cut into slices issue x first (x-first issue order; the same
//    sweep: 12.7-12.8 us without it);
//  * sparse rows of 4 or 5 chunks a lane at 3 or 4 vectors, unsliced: two
//    rows a wave (row pairs), when that still gives two blocks per CU; at
//    these batch sizes the VALU kernel is bound by instruction issue, and a
//    pair shares the wave's fixed work and its x reads (Qwen3-32B gate+up at
//    4 vectors 61.8 -> 53.3 us; at 2 vectors no gain and at one a loss, so
//    not taken there; NMSPMV_RPW=2 takes them from one vector; pairs: false
//    keeps one row a wave, for the fused hybrid launch).
inline bool plan_rowslice(int64_t R, int64_t C, bool dense, bool glu, int B, Plan* P, bool pairs = true)
{
    const int cus = cu_count();
    // Long rows on one wave (up to 16 chunks a lane: a single vector,
    // sparse, not gated), when NMSPMV_MAX_CPL asks for it.
    const int max_cpl = (B == 1 && !dense && !glu && g_env.max_cpl > 8) ? std::min(g_env.max_cpl, 16) : 8;
    int S = 1, rpb = dense ? 4 : 8;
    if (C > (dense ? 8 : 5) * kWave && C > (int64_t)max_cpl * kWave) {
        const int64_t max_cps = (dense ? 7 : 8) * kWave;
        S = 2;
        while (S < 16 && (C + S - 1) / S > max_cps)
            S *= 2;
        rpb = std::max(1, 8 / S);
    }
    while (S < 16 && R * S < 16LL * cus && (C + 2 * S - 1) / (2 * S) >= kWave) {
        S *= 2;
        rpb = std::max(1, 8 / S);
    }
    if (g_env.slices > 0)
        S = 1 << log2_exact(std::min(g_env.slices, 16));
    if (glu && S > 8)                            // gated rows come in pairs: at least 2 rows per block
        S = 8;
    const int64_t cps = (C + S - 1) / S;
    const int cpl = (int)((cps + kWave - 1) / kWave);
    if (cpl > max_cpl)
        return false;
    while (rpb > 1 && (R + rpb - 1) / rpb < 2 * cus)
        rpb /= 2;
    if (g_env.rpb > 0)
        rpb = g_env.rpb;
    if (glu)
        rpb = std::max(2, rpb & ~1);
    if (rpb * S > 16)
        return false;
    const int64_t threads = (int64_t)rpb * S * kWave;
    int rpw = 1;
    // (a single vector's x must fit one register unit a thread: the pair kernels are built for that)
    if (pairs && !dense && S == 1 && B >= (g_env.rpw == 2 ? 1 : 3) && B <= 4 && (cpl == 4 || cpl == 5) &&
        g_env.rpw != 1 && g_env.rpb == 0 && (R + 2 * rpb - 1) / (2 * rpb) >= 2 * cus &&
        (B > 1 || 2 * C <= threads))
        rpw = 2;
    P->kind = 1;
    P->S = S;
    P->ls = log2_exact(S);
    P->xf = g_env.xfirst >= 0 ? (g_env.xfirst != 0) : (S >= 2);
    P->rpw = rpw;
    P->rpb = rpb * rpw;
    P->cpl = cpl;
    P->threads = (int)threads;
    P->grid = (unsigned)((R + P->rpb - 1) / P->rpb);
    return true;
}

// Chooses the kernel for a matrix shape: the row-slice kernel when x fits its
// LDS budget and rows are at most 1600 chunks (sparse, K <= 25600) or 3200
// chunks (dense, K <= 25600); otherwise the stream kernel -- whose blocks
// stage x once for many rows -- with x in K-tiles when it exceeds the budget.
// (Single-vector timing, us, stream -> row-slice: Qwen3-32B down, 5120 x
// 25600, 2:4 32.8 -> 28.8 and dense 50.9 -> 44.7; Llama-3.3-70B down, 8192 x
// 28672, 2:4 47.6 -> 50.4 and dense 78.0 -> 84.7.)
template <int F>
Plan plan_for(int64_t R, int64_t K, int B, bool glu, bool pairs = true)
{
    std::call_once(g_env_once, read_env);
    constexpr int COLS = chunk_cols<F>();
    const int64_t C = K / COLS;
    const size_t tab = (size_t)table_units<F>() * kUnitBytes;
    const size_t xbytes = (size_t)B * (size_t)x_row_units(K) * 16;   // x as staged (rows rounded to 64 units)
    const bool fits = xbytes <= (size_t)kXTileBudget;
    Plan P;
    int kind = g_env.kernel;
    if (kind != 1 && kind != 3)
        kind = (fits && C <= (F == kDense ? 50 : 25) * kWave) ? 1 : 3;
    if (kind == 1 && fits && plan_rowslice(R, C, F == kDense, glu, B, &P, pairs)) {
        P.lds = tab + xbytes + (size_t)P.rpb * P.S * B * 4;
        if (g_env.blocks_per_cu >= 2 && g_env.blocks_per_cu <= 8)
            P.lds = std::max(P.lds, (size_t)kLdsMax / (g_env.blocks_per_cu + 1) + 256);
        return P;
    }
    const int cus = cu_count();
    P.kind = 3;
    // Two 512-thread blocks per CU; x larger than the tile budget is cut into
    // equal K-tiles of whole 1024-column units (each tile costs a barrier and
    // an x restage per block).
    int threads = 512;
    if (g_env.threads > 0 && g_env.threads <= 1024 && g_env.threads % kWave == 0)
        threads = g_env.threads;
    P.threads = threads;
    const int nw = P.threads / kWave;
    // Rows per wave as the kernel counts them (gated rows go to waves in pairs).
    const int per = glu ? 2 : 1;
    const int64_t Ru = R / per;
    int64_t blocks = g_env.blocks > 0 ? g_env.blocks : 2LL * cus;
    while (blocks > 1 && (blocks - 1) * nw >= Ru)
        --blocks;
    const int64_t budget = g_env.tile_bytes > 0 ? g_env.tile_bytes : kXTileStream;
    int64_t tile = K;
    if ((int64_t)B * K * 2 > budget) {
        const int64_t ntiles = ((int64_t)B * K * 2 + budget - 1) / budget;
        tile = ((K + ntiles - 1) / ntiles + 1023) / 1024 * 1024;
        if (tile >= K)
            tile = K;
    }
    // With several tiles each wave keeps its rows' partial sums in LDS: more
    // blocks when that would take more than 16 KB, narrower tiles if the
    // block would still exceed the CU's LDS.
    int64_t rpw = per * ((Ru + blocks * nw - 1) / (blocks * nw));
    if (tile < K) {
        const int64_t rpw_max = std::max<int64_t>(per, (16 * 1024) / ((int64_t)nw * B * 4));
        if (rpw > rpw_max) {
            blocks = (Ru + nw * (rpw_max / per) - 1) / (nw * (rpw_max / per));
            rpw = per * ((Ru + blocks * nw - 1) / (blocks * nw));
        }
        while (tile > 1024 && tab + (size_t)B * x_row_units(tile) * 16 + (size_t)nw * rpw * B * 4 > (size_t)kLdsMax)
            tile -= 1024;
    }
    P.tile_cols = (int)tile;
    P.grid = (unsigned)blocks;
    P.lds = tab + (size_t)B * (size_t)x_row_units(tile) * 16 + (tile < K ? (size_t)nw * rpw * B * 4 : 0);
    return P;
}

// Row-slice x staging: 1 = one register per thread covers B x K (each thread
// loads one 16-byte unit and stores it to LDS); 4 = four registers a thread
// cover a single vector (not with more than 8 chunks a lane, whose weights
// already hold most of the registers); 0 = global-to-LDS loads, which hold no
// registers.
inline int rowslice_x_regs(int B, int64_t K, int threads, int cpl)
{
    std::call_once(g_env_once, read_env);
    const int64_t xunits = (int64_t)B * (K / 8);
    if (xunits <= threads)
        return 1;
    return (B == 1 && xunits <= 4LL * threads && g_env.xdma != 1 && cpl <= 8) ? 4 : 0;
}

// Fused hybrid launch (a hybrid matrix's RS sparse and its dense rows in one
// row-slice launch, B of 1 to 3): the sparse rows' row-slice plan with an
// even number of rows per block; the dense rows then take half as many rows
// per block over twice the slices (same threads, same chunks per lane).
// Where the sparse plan went to one row per block to keep two blocks per CU,
// the dense rows' blocks add to the launch, so it takes two rows per block
// (and the LDS for their partial sums).  false: no fused launch.
template <int F>
bool plan_hybrid(int64_t RS, int64_t K, int B, Plan* out)
{
    Plan P = plan_for<F>(RS, K, B, false, false);
    if (P.kind == 1 && P.rpb == 1 && g_env.rpb == 0 && P.S <= 8) {
        P.rpb = 2;
        P.threads = 2 * P.S * kWave;
        P.grid = (unsigned)((RS + 1) / 2);
        P.lds = (size_t)table_units<F>() * kUnitBytes + (size_t)B * x_row_units(K) * 16 + (size_t)P.rpb * P.S * B * 4;
    }
    if (P.kind != 1 || P.rpb < 2 || P.rpb % 2 != 0 || P.cpl > 8)
        return false;
    *out = P;
    return true;
}

// Whether a batch goes to the matrix-core kernels rather than the VALU ones
// (timing on MI355X at the Qwen3-32B MLP shapes with weights streamed from
// HBM).  The LDS-ring kernel wins from 5 vectors (sparse) over the row-slice
// kernel and from 3 where x is too long for it and the VALU path would be
// the K-tiled stream kernel; dense from 4 either way; the staged kernel
// (sparse rows with K % 32 != 0) from 6.  Above 8 vectors only the matrix
// cores take the batch.  NMSPMV_MFMA_MIN_B overrides the threshold.
template <int F>
bool use_mfma(int64_t R, int64_t K, int B, bool glu)
{
    std::call_once(g_env_once, read_env);
    if (B > kVectorMaxBatch)
        return true;
    if (g_env.mfma_min_b > 0)
        return B >= g_env.mfma_min_b;
    const bool dense = F == kDense;
    if (!dense && K % 32 != 0)
        return B >= 6;
    if (dense)
        return B >= 4;
    return B >= (plan_for<F>(R, K, B, glu).kind == 3 ? 3 : 5);
}

// Staged matrix-core launch shape: 16-row tiles; 1, 2, 4 or 8 K-slices (each
// at least one 32-chunk stage) until the launch has ~12 waves per CU (the
// kernel's register use allows 3 per SIMD); the slices of a tile, or 4 tiles,
// share a block of at most 8 waves.  With two batch tiles (17 to 32 vectors)
// at most 2 slices, and 1 from 24 vectors when there are more tiles than
// CUs.  Measured with bf16 2:4 rows on shapes from 1024 x 4096 to
// 8192 x 28672: 2 slices beat 4 and 8 on every shape at 17 and 32 vectors
// (by 4-30%; 4096 x 4096 at 32: 16.0 against 22.8 us with 8); at 24-32
// vectors 1 slice beat 2 by 6-11% on every shape of more than 256 tiles
// (5120 x 25600 at 32: 104.6 against 117.3 us) and lost by 16-42% on those
// of 256 or fewer; at 17 vectors it lost on all.
template <int F>
Plan plan_mfma_stage(int64_t R, int64_t K, int NT, int B)
{
    std::call_once(g_env_once, read_env);
    constexpr int COLS = chunk_cols<F>();
    const int cus = cu_count();
    const int64_t C = K / COLS, tiles = (R + 15) / 16;
    int S = 1;
    const int smax = NT == 2 ? (B >= 24 && tiles > cus ? 1 : 2) : 8;
    while (S < smax && tiles * S < 12LL * cus && C / (2 * S) >= kStageChunks)
        S *= 2;
    if (g_env.mfma_slices > 0 && g_env.mfma_slices <= 8)
        S = g_env.mfma_slices;
    int tpb = std::max(1, 4 / S);
    while (tpb > 1 && (tiles + tpb - 1) / tpb < 2 * cus)
        tpb /= 2;
    Plan P;
    P.kind = 5;
    P.S = S;
    P.rpb = tpb;
    P.threads = S * tpb * kWave;
    P.grid = (unsigned)((tiles + tpb - 1) / tpb);
    const size_t waves = (size_t)S * tpb;
    P.lds = (size_t)mfma_table_units<F>() * kUnitBytes + waves * kStageBytes + waves * NT * kWave * 4 * sizeof(float);
    return P;
}

// LDS-ring launch shape (rules from sweeps on MI355X at the Qwen3-32B MLP
// shapes, weights streamed from HBM): 16-row tiles, one per wave up to 8
// vectors, two above (x, then 16 rows per stage, serves both; four tiles a
// wave, tried for sparse rows above 16, double the LDS a wave holds and halve
// the waves a CU keeps -- slower than two tiles with x shared by two waves);
// a block holds one wave group, its K split into S
// stage-interleaved slices (one wave each).  S is the largest power of two
// (each slice keeping at least four stages, at most 8 waves a block, the
// kernel's launch bound) whose launch still fits the CUs' LDS in one round:
// a second, partly filled round costs more than the extra waves gain.
template <int F>
Plan plan_mfma_ring(int64_t R, int64_t K, int B)
{
    std::call_once(g_env_once, read_env);
    constexpr int COLS = chunk_cols<F>();
    const int cus = cu_count();
    const int64_t C = K / COLS, NS = (C + kStageChunks - 1) / kStageChunks;
    int TW = B > 8 ? 2 : 1;
    if (B <= 16 && (g_env.ring_tiles == 1 || g_env.ring_tiles == 2))
        TW = g_env.ring_tiles;                   // above 16 vectors the tile count is fixed
    const int64_t tiles = (R + 16 * TW - 1) / (16 * TW);
    const size_t tab = (size_t)mfma_table_units<F>() * kUnitBytes;
    const size_t ring = 2 * (size_t)(TW == 2 ? ring_slot_bytes<F, 2>(B) : ring_slot_bytes<F, 1>(B));
    const int wmax = (int)std::min<size_t>(8, (kLdsMax - tab) / ring);
    // Waves resident at once with S-wave blocks (LDS-bound).
    auto resident = [&](int S) { return (int64_t)(kLdsMax / (tab + S * ring)) * S * cus; };
    int S = 1;
    for (int s2 = 2; s2 <= wmax && NS >= 4LL * s2; s2 *= 2)
        if (tiles * s2 <= resident(s2))
            S = s2;
    if (g_env.mfma_slices > 0 && g_env.mfma_slices <= wmax)
        S = g_env.mfma_slices;
    Plan P;
    P.kind = 6;
    P.S = S;
    P.rpb = 1;
    P.cpl = TW;
    P.threads = S * kWave;
    P.grid = (unsigned)tiles;
    P.lds = tab + (size_t)S * ring;
    // One slice per tile: up to 4 waves (one tile group each) share a block's
    // staged x (2 with two tiles per wave), while the launch keeps at least
    // one block per CU.
    // (A share set by NMSPMV_RING_SHARE is also cut to what the CU's LDS holds.)
    const size_t wring = 2 * (size_t)TW * (kRingValues + (F == kDense ? 0 : kRingMasks));
    const size_t xslot = (size_t)ring_x_rows<F>(B) * ring_x_units<F>() * 16;
    int W = TW == 1 ? 4 : 2;
    if (g_env.ring_share > 0)
        W = std::min(g_env.ring_share, 8);
    while (W > 1 && ((tiles + W - 1) / W < cus || tab + W * wring + 2 * xslot > (size_t)kLdsMax))
        W /= 2;
    // Blocks past what the CUs hold at once run as a second round, and each
    // block streams its tiles' whole K, so the launch lasts about as long as
    // the busiest CU's tiles: ceil(blocks / CUs) blocks of W tiles each.
    // When the share above leaves such a round, take the share with the
    // fewest tiles on the busiest CU (the widest on a tie: less x staged),
    // keeping every CU busy and 12 waves a CU in flight (the kernel's
    // registers allow about 20 with one tile a wave).  Qwen3-32B gate+up at 8
    // vectors (51200 x 5120, 3200 tiles), tiles on the busiest CU and time by
    // share: 3: 15, 73.8 us; 4: 16, 75.1; 5: 15, 72.0; 6: 18, 77.0; 7: 14,
    // 65.9.  With two tiles a wave (above 8 vectors) the default share stays:
    // at 16 vectors the same matrix took 89.2 us at two a block (8 tile pairs
    // on the busiest CU) and 90.3 at seven (7, but one block of 7 waves a CU).
    auto per_cu = [&](int w) -> int64_t {
        const size_t l = tab + w * wring + 2 * xslot;
        return l > (size_t)kLdsMax ? 0 : std::min<int64_t>((int64_t)(kLdsMax / l), 20 / w);
    };
    if (g_env.ring_share <= 0 && S == 1 && W > 1 && TW == 1) {
        auto load = [&](int w) { return ((tiles + w - 1) / w + cus - 1) / cus * w; };
        if ((tiles + W - 1) / W > per_cu(W) * cus) {
            int best = W;
            for (int w = 2; w <= 8; ++w) {
                const int64_t nb = per_cu(w), blocks = (tiles + w - 1) / w;
                if (nb == 0 || blocks < cus || std::min<int64_t>(nb, (blocks + cus - 1) / cus) * w < 12)
                    continue;
                if (load(w) < load(best) || (load(w) == load(best) && w > best && best != W))
                    best = w;
            }
            W = best;
        }
        // CU-major tile map: k blocks on every CU in one round, CU c's
        // ceil or floor of tiles / CUs split over them, so the busiest CU
        // holds ceil(tiles / CUs) tiles instead of ceil(blocks / CUs) full
        // blocks.  The fewest blocks a CU (fewest idle waves) that keep 8
        // waves a CU.  Qwen3-32B gate+up at 8 vectors (3200 tiles): two
        // blocks of 6-7 tiles a CU, 13 tiles on the busiest CU against 14.
        const int64_t even = (tiles + cus - 1) / cus;
        for (int k = 1; k <= 4; ++k) {
            const int64_t wb = (even + k - 1) / k;
            if (wb < 2 || wb > 8 || per_cu((int)wb) < k || k * wb < 8)
                continue;
            if (even < load(W)) {
                W = (int)wb;
                P.map_k = k;
                P.map_cus = cus;
            }
            break;
        }
    }
    if (S == 1 && W > 1) {
        P.kind = 7;
        P.rpb = W;
        P.threads = W * kWave;
        P.grid = P.map_k ? (unsigned)(P.map_k * cus) : (unsigned)((tiles + W - 1) / W);
        P.lds = tab + W * wring + 2 * xslot;
    }
    return P;
}

// The LDS-ring kernel takes dense rows at any batch, and sparse rows whose
// mask row is a whole number of dwords (K % 32 == 0): up to 16 vectors
// always, above 16 when there is at least one 64-row block (two waves of two
// tiles sharing x) per CU (measured: with fewer the ring needs K-slices,
// whose waves cannot share x, and does no better than the staged kernel).  Other sparse batches run on the staged
// kernel, where up to 16 vectors are one tile of the matrix cores' batch
// dimension and 17 to 32 take two, both fed by the same weight loads.
template <int F>
bool mfma_use_ring(int64_t R, int64_t K, int B)
{
    std::call_once(g_env_once, read_env);
    const bool ring_fits = F == kDense || (K % 32 == 0 && (B <= 16 || R >= 64LL * cu_count() || g_env.kernel == 6));
    return ring_fits && g_env.kernel != 5;
}

// Workspace of the K-split ring plan: partial sums, then one counter per tile
// group (zero between launches).
constexpr size_t kSplitPartBytes = size_t(16) << 20;
constexpr int kSplitMaxGroups = 16384;
constexpr size_t kSplitWorkspaceBytes = kSplitPartBytes + size_t(kSplitMaxGroups) * 4;

// K-split ring plan (kind 8), for the calls that bring a workspace: where the
// LDS-ring plan would cut each 16-row tile into per-wave K-slices (few tiles
// for the CUs, so each wave stages its own x: about as many x bytes as
// weight bytes at 8 vectors), blocks of W waves (one tile group, TW tiles a
// wave) share each staged x over one of KS contiguous stage ranges instead,
// and the last block of a group adds the KS partial sums.  A CU's share of
// the read bandwidth sets the pace (a block on a CU that holds three streams
// a third slower than one on a CU that holds two), so W and KS are chosen for
// the least bytes on the busiest CU: ceil(blocks / CUs) blocks, each staging
// its W units and one x per stage over ceil(stages / KS) stages, plus two
// stages' worth for the block's start (every block issues its first loads at
// once; they land after ~4 us), the widest W on a tie; at least 4 stages a
// split, 4 waves a CU, and a block's LDS within a CU's.  Qwen3-32B down, 5120 x 25600, 8
// vectors (W, KS: that figure, us on one GPU): 2, 4: 1078 KB, 42.3; 2, 8:
// 998 KB, 42.3; 3, 8: 1075 KB, 44.5; 5, 8: 814 KB, 40.5; 5, 4: 733 KB, 40.3
// (one block a CU).  false: keep the ring plan.
template <int F>
bool plan_mfma_split(int64_t R, int64_t K, int B, Plan* out)
{
    std::call_once(g_env_once, read_env);
    if (g_env.splitk == 1)
        return false;
    const Plan base = plan_mfma_ring<F>(R, K, B);
    constexpr int COLS = chunk_cols<F>();
    const int cus = cu_count();
    const int TW = base.cpl;
    const int NT = B > 16 ? 2 : 1;
    const int64_t C = K / COLS, NS = (C + kStageChunks - 1) / kStageChunks;
    const int64_t tiles = (R + 16 * TW - 1) / (16 * TW);
    // Only for short matrices: fewer than four tile units a CU, where the
    // ring plan cuts tiles into K-slices.  With more tiles the ring plan's
    // blocks fill the CUs (the dense 25600 x 5120 gate at 4 vectors, 1600
    // tiles: 49.6 us on the ring plan, 65.6 on a K-split of 1280 ten-stage
    // blocks).
    if (g_env.splitk != 2 && !(base.kind == 6 && base.S >= 2 && tiles < 4LL * cus))
        return false;
    const size_t tab = (size_t)mfma_table_units<F>() * kUnitBytes;
    const size_t unit = (size_t)TW * (kRingValues + (F == kDense ? 0 : kRingMasks));   // a unit's stage
    const size_t xslot = (size_t)ring_x_rows<F>(B) * ring_x_units<F>() * 16;
    const int ks_env = g_env.splitk_ks >= 2 && g_env.splitk_ks <= 32 ? (int)std::min<int64_t>(g_env.splitk_ks, NS) : 0;
    int W = 0, KS = 0;
    double best = 0.0;
    for (int w = 1; w <= 8; ++w) {
        if (g_env.ring_share > 0 && w != std::min(g_env.ring_share, 8))
            continue;
        const size_t lds = tab + w * 2 * unit + 2 * xslot;
        if (lds > (size_t)kLdsMax)
            break;
        const int64_t groups = (tiles + w - 1) / w;
        for (int ks = 2; ks <= 32; ++ks) {
            if (ks_env ? ks != ks_env : NS < 4LL * ks)
                continue;
            if (groups > kSplitMaxGroups || (size_t)ks * (size_t)groups * w * TW * NT * 1024 > kSplitPartBytes)
                continue;
            const int64_t per_cu = (groups * ks + cus - 1) / cus;
            if (g_env.ring_share <= 0 && !ks_env && std::min<int64_t>(per_cu, (int64_t)(kLdsMax / lds)) * w < 4)
                continue;                        // too few waves a CU to cover the loads' latency
            const double bytes = (double)per_cu * (double)((NS + ks - 1) / ks + 2) * (double)(w * unit + xslot);
            if (!W || bytes < best || (bytes == best && w > W)) {
                best = bytes;
                W = w;
                KS = ks;
            }
        }
    }
    if (!W)
        return false;
    const int64_t groups = (tiles + W - 1) / W;
    const int64_t stages = (NS + KS - 1) / KS;
    if ((size_t)KS * (size_t)groups * W * TW * NT * 1024 > kSplitPartBytes)
        return false;
    Plan P;
    P.kind = 8;
    P.S = 1;
    P.rpb = W;
    P.cpl = TW;
    P.threads = W * kWave;
    P.grid = (unsigned)(groups * KS);
    P.ks = KS;
    P.kstages = (int)stages;
    P.lds = tab + W * 2 * unit + 2 * xslot;
    *out = P;
    return true;
}

// The K-split plan (calls with a workspace) takes the ring kernel's rows --
// dense rows, and sparse rows whose mask row is a whole number of dwords --
// at any batch, also where the plain call would take the staged kernel
// (sparse, above 16 vectors, on few rows): its blocks share x across tiles,
// which the ring's K-slices cannot.
template <int F>
bool mfma_use_split(int64_t R, int64_t K, int B, Plan* out)
{
    std::call_once(g_env_once, read_env);
    return (F == kDense || K % 32 == 0) && g_env.kernel != 5 && plan_mfma_split<F>(R, K, B, out);
}

}  // namespace nmh

#endif  // NM_PLAN_H
