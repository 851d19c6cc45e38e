// nmspmv.hip -- libnmspmv: N:M sparse matrix-vector products on gfx950.
//
// The decode-time hot path named by "SparseDecoding: Decoding-Aware Pruning
// for Accurate and Efficient LLM Inference" (humanity-list story page,
// "Abstract"): a product of an N:M-pruned weight with one activation vector,
// where a per-column bit marks which weights were kept and each group's kept
// values sit at a constant offset; decoding is memory-bound, so the weight
// bytes read per token set the time.  The pages' kernel was written for A100;
// this one is designed for CDNA4 (wave64, 160 KB LDS per CU, HBM3E) and shares
// no code with the CPU oracle that the tests compare it against.
//
// Format (include/nmspmv.h): values [R][K*N/M] 16-bit, group g of a row at
// value g*N; masks [R][K/8], one bit per dense column, LSB first.
//
// Work unit: a 16-byte chunk of a row -- 8 weights (dense) or, at N/M = 1/2,
// 8 kept values covering 16 dense columns with their 16 mask bits (2 bytes,
// at the same chunk index in the mask row: fixed step, no index arrays).
// Lanes stream chunks with 128-bit non-temporal loads; x sits in LDS.
//   2:4  each mask nibble is one group: a 16-entry LDS table turns it into a
//        byte-permute selector that gathers the group's two x halves next to
//        each other, and one packed dot2 multiplies them with the group's two
//        values (x-select).
//   4:8  each mask byte is one group: a 256-entry LDS table gives four
//        selectors that spread the group's four values over its eight dense
//        columns, then four dot2 with contiguous x (value expansion).
//   dense  four dot2 per chunk.
// Products of two 16-bit floats are exact in fp32; sums are fp32; each row is
// reduced across the 64 lanes with DPP row permutes and four lane reads in a
// fixed order (deterministic), then rounded once to fp16/bf16.
//
// Kernel shapes (chosen per matrix shape on the host):
//   rowslice_kernel  a wave owns one (row, K-slice) item and issues all of its
//                    loads before anything else; many short-lived waves.
//   hybrid_rowslice_kernel  a hybrid matrix's sparse and dense rows in one
//                    launch: two row-slice plans side by side.
//   stream_kernel    waves walk rows g, g+G, ... with the next group of loads
//                    in flight while computing (long rows, few blocks); x in
//                    K-tiles when B*K*2 bytes exceed the LDS tile.
//   generic_spmv_kernel  any N:M with M in {4, 8} and K % 8 == 0 (untuned).
//   mfma_ring_kernel  batches of a few vectors and up: 16-row tiles of W times
//                    x^T on the matrix cores (v_mfma_f32_16x16x32), the packed
//                    values expanded to the operand in registers; weights,
//                    masks and x streamed into a per-wave LDS ring by
//                    global-to-LDS loads.
//   mfma_stage_kernel  the same product with the weights staged through
//                    registers (sparse rows with K % 32 != 0, and sparse
//                    batches above 16 on matrices too short for the ring).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "nm_decode.h"
#include "nm_launch.h"
#include "nm_plan.h"
#include "nmspmv.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

using namespace nmh;   // layout constants, formats, launch planning and argument rules

// ---- arithmetic helpers ----------------------------------------------------

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);

template <>
__device__ __forceinline__ float dot2<NM_FP16>(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

template <>
__device__ __forceinline__ float dot2<NM_BF16>(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int DT>
__device__ __forceinline__ float to_f32(uint16_t bits)
{
    if constexpr (DT == NM_FP16)
        return (float)__builtin_bit_cast(_Float16, bits);
    else
        return __builtin_bit_cast(float, (uint32_t)bits << 16);
}

// fp32 -> 16-bit, round to nearest even (v_cvt_f16_f32 / v_cvt_pk_bf16_f32).
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float v)
{
    if constexpr (DT == NM_FP16)
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    else
        return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes; every lane must be active.  Within each row of 16
// lanes: swap neighbours, swap pairs, mirror halves, mirror the row; then the
// four row sums are read out and added in a fixed order.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (a + b) + (c + d);
}

// ---- selector tables ---------------------------------------------------------

// 2:4.  Nibble n marks the kept columns j0 < j1 of a 4-column group whose x
// halves sit in the 8-byte source {x23 : x01} (half j in bytes 2j, 2j+1).  The
// selector moves x[j0] to the low half and x[j1] to the high half, matching
// the order of the group's two stored values.  Nibbles without exactly two
// bits are malformed; their selector yields zeros (0x0C = zero byte).
__device__ uint32_t select24(uint32_t n)
{
    if (__builtin_popcount(n) != 2)
        return 0x0C0C0C0Cu;
    const uint32_t j0 = __builtin_ctz(n);
    const uint32_t j1 = 31 - __builtin_clz(n);
    return (2 * j0) | ((2 * j0 + 1) << 8) | ((2 * j1) << 16) | ((2 * j1 + 1) << 24);
}

// 4:8, one nibble of a group's mask byte (every kernel's 4:8 table): the
// selectors of the nibble's two dense dwords (columns 2d, 2d+1 of its four)
// over {hi dword : lo dword} of the group's four values (in column order,
// value k in bytes 2k, 2k+1), copying value k into a kept column and zero
// bytes (0x0C) elsewhere, the nibble's first kept value being value k0.  The low nibble's values come first (k0 = 0); in a group with
// exactly four kept columns the high nibble's follow them, so its k0 is
// 4 - popcount(high nibble) and each nibble's selectors depend on that nibble
// alone: two 16-entry tables of 8-byte entries (128 bytes each, every entry
// on its own two LDS banks) instead of one 256-entry table of 16-byte
// entries, whose look-ups from 64 lanes fell on the same banks.  A malformed
// mask gives junk selector bytes, never an out-of-range access.
__device__ u32x2 select48_nibble(uint32_t n, uint32_t k0)
{
    uint32_t s[2];
    uint32_t k = k0;
    for (int d = 0; d < 2; ++d) {
        uint32_t sel = 0;
        for (int h = 0; h < 2; ++h) {
            uint32_t pair = 0x0C0Cu;
            if ((n >> (2 * d + h)) & 1u) {
                pair = (2 * k) | ((2 * k + 1) << 8);
                ++k;
            }
            sel |= pair << (16 * h);
        }
        s[d] = sel;
    }
    return u32x2{s[0], s[1]};
}

template <int F>
__device__ __forceinline__ void build_table(u32x4* tab)
{
    if constexpr (F == kNM24) {
        if (threadIdx.x < 4)
            tab[threadIdx.x] = u32x4{select24(4 * threadIdx.x), select24(4 * threadIdx.x + 1),
                                     select24(4 * threadIdx.x + 2), select24(4 * threadIdx.x + 3)};
    } else if constexpr (F == kNM48) {
        // entries 0-15: low nibbles; 16-31: high nibbles
        u32x2* t2 = reinterpret_cast<u32x2*>(tab);
        for (unsigned i = threadIdx.x; i < 32; i += blockDim.x)
            t2[i] = i < 16 ? select48_nibble(i, 0) : select48_nibble(i - 16, 4u - __builtin_popcount(i - 16));
    }
}

// Global-to-LDS loads (gfx950): a load instruction's LDS destination is its
// base (M0) + 16 bytes x lane; the kernels that use them declare no static
// LDS, so dynamic LDS starts at offset 0.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

template <int BYTES>
__device__ __forceinline__ void load_to_lds(const void* g, uint32_t lds_offset)
{
    static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte lanes");
#if defined(__HIP_DEVICE_COMPILE__)
    lds_void_t* dst = (lds_void_t*)((lds_u8_t*)nullptr + lds_offset);
    if constexpr (BYTES == 16)
        __builtin_amdgcn_global_load_lds(g, dst, 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(g, dst, 4, 0, 0);
#else
    (void)g;
    (void)lds_offset;
#endif
}

// s_waitcnt with vmcnt <= N (N < 64) and the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt with vmcnt <= N and lgkmcnt 0.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// x in LDS: [NB][bstride] 16-byte units, bstride a multiple of 64.  Sparse
// formats keep each 64-unit run of a batch row as two 32-slot halves, its
// even units first (unit 64 q + 2 i at slot 64 q + i, unit 64 q + 2 i + 1 at
// slot 64 q + 32 + i), so that lanes reading the two units of consecutive
// chunks touch consecutive LDS addresses, and one 64-lane global-to-LDS load
// (1 KB, lane l at slot 64 q + l) fills a whole run.  Dense rows keep unit
// order.
template <int F>
__device__ __forceinline__ int x_slot(int b, int j, int bstride)
{
    if constexpr (F == kDense)
        return b * bstride + j;
    else
        return b * bstride + (j & ~63) + ((j & 1) << 5) + ((j >> 1) & 31);
}

// Slot of the first unit of sparse chunk c (its second unit is 32 slots on).
__device__ __forceinline__ int x_chunk_slot(int c)
{
    return ((c >> 5) << 6) + (c & 31);
}

// The byte offset of a dynamic-LDS pointer (dynamic LDS starts at 0 in these
// kernels, which declare no static LDS).
__device__ __forceinline__ uint32_t lds_offset_of(const void* p)
{
    return (uint32_t)(uintptr_t)p;
}

// x [NB][K] into LDS at byte offset x_base, laid out by x_slot<F> with
// bstride units per batch row: one 64-lane global-to-LDS load per 64-unit
// run (lanes past the end of a row reload the row's unit 0 into slots no
// chunk reads), the runs dealt round-robin over the block's waves.  x takes
// no registers on the way; a wave's loads count in vmcnt like any other, so
// a wave that has issued n loads after these knows them complete at
// vmcnt <= n, and the block meets at a barrier before reading x.
template <int F, int NB>
__device__ __forceinline__ void x_dma(const u32x4* __restrict__ x4, int K, int bstride, uint32_t x_base, int wave,
                                      int nwaves, int lane)
{
    const int units = K >> 3;
    const int per_row = (units + 63) >> 6;
    const int lj = F == kDense ? lane : 2 * (lane & 31) + (lane >> 5);
    for (int g = wave; g < NB * per_row; g += nwaves) {
        const int b = NB == 1 ? 0 : g / per_row;
        const int q = g - b * per_row;
        const int j = 64 * q + lj;
        load_to_lds<16>(x4 + (size_t)b * units + (j < units ? j : 0), x_base + (uint32_t)(b * bstride + 64 * q) * 16);
    }
}

// The stream kernel stages x in tiles, in two halves around its first weight
// loads: x_fetch_tile issues this thread's first kXU units of a tile (all of
// it when the tile has at most kXU * blockDim units) into registers before
// the weight loads are issued; x_store_tile writes them to LDS, and the
// rest, if any, straight through.  Loads retire in issue order, so a wave
// can store its x and reach the block barrier while its weight loads are
// still in flight.  The loads are branch-free (lanes past the end of the
// tile reload unit 0) so that the compiler can count them exactly; only the
// LDS stores are predicated.
constexpr int kXU = 4;    // x registers of the stream kernel (per tile)

// A tile of `cols` columns starting at column c0.
template <int NB>
__device__ __forceinline__ void x_fetch_tile(const u32x4* __restrict__ x4, int K, int c0, int cols, u32x4* xr)
{
    const int q = cols / 8, n = NB * q;
#pragma unroll
    for (int u = 0; u < kXU; ++u) {
        int i = threadIdx.x + u * blockDim.x;
        i = i < n ? i : 0;
        const int b = NB == 1 ? 0 : i / q;      // (NB == 1: i < q whenever it is used)
        xr[u] = x4[(size_t)b * (K / 8) + c0 / 8 + (i - b * q)];
    }
}

template <int F, int NB>
__device__ __forceinline__ void x_store_tile(u32x4* xs, const u32x4* __restrict__ x4, int K, int c0, int cols,
                                             int bstride, const u32x4* xr)
{
    const int q = cols / 8, n = NB * q;
#pragma unroll
    for (int u = 0; u < kXU; ++u) {
        const int i = threadIdx.x + u * blockDim.x;
        const int b = NB == 1 ? 0 : i / q;      // (NB == 1: i < q whenever it is used)
        if (i < n)
            xs[x_slot<F>(b, i - b * q, bstride)] = xr[u];
    }
    for (int i = threadIdx.x + kXU * blockDim.x; i < n; i += blockDim.x) {
        const int b = NB == 1 ? 0 : i / q;      // (NB == 1: i < q whenever it is used)
        xs[x_slot<F>(b, i - b * q, bstride)] = x4[(size_t)b * (K / 8) + c0 / 8 + (i - b * q)];
    }
}

// ---- one 16-byte chunk -------------------------------------------------------

// The LDS slot of staged x that chunk c (of the staged columns) starts at:
// its unit (dense) or its first unit (sparse; the second is 32 slots on).
template <int F>
__device__ __forceinline__ int chunk_xslot(int c)
{
    if constexpr (F == kDense)
        return c;
    else
        return x_chunk_slot(c);
}

// The slot step between chunks c and c + 64 (same lane, next load slot).
template <int F>
constexpr int xslot_step()
{
    return F == kDense ? 64 : 128;
}

// acc[b] += (chunk . x[b][chunk columns]).  xs: staged x, xslot: the chunk's
// x slot (chunk_xslot), bstride: units per batch row.
template <int F, int DT, int NB>
__device__ __forceinline__ void chunk_dot(const u32x4 v, const uint32_t mk, const u32x4* __restrict__ tab,
                                          const u32x4* __restrict__ xs, const int xslot, const int bstride, float* acc)
{
    if constexpr (F == kDense) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x4 xa = xs[b * bstride + xslot];
            float a = acc[b];
            a = dot2<DT>(v.x, xa.x, a);
            a = dot2<DT>(v.y, xa.y, a);
            a = dot2<DT>(v.z, xa.z, a);
            a = dot2<DT>(v.w, xa.w, a);
            acc[b] = a;
        }
    } else if constexpr (F == kNM24) {
        const uint32_t* t = reinterpret_cast<const uint32_t*>(tab);
        const uint32_t s0 = t[mk & 0xF], s1 = t[(mk >> 4) & 0xF], s2 = t[(mk >> 8) & 0xF], s3 = t[(mk >> 12) & 0xF];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x4 xa = xs[b * bstride + xslot];
            const u32x4 xb = xs[b * bstride + xslot + 32];
            float a = acc[b];
            a = dot2<DT>(v.x, __builtin_amdgcn_perm(xa.y, xa.x, s0), a);
            a = dot2<DT>(v.y, __builtin_amdgcn_perm(xa.w, xa.z, s1), a);
            a = dot2<DT>(v.z, __builtin_amdgcn_perm(xb.y, xb.x, s2), a);
            a = dot2<DT>(v.w, __builtin_amdgcn_perm(xb.w, xb.z, s3), a);
            acc[b] = a;
        }
    } else {
        const u32x2* t2 = reinterpret_cast<const u32x2*>(tab);
        const u32x2 a0 = t2[mk & 0xF], a1 = t2[16 + ((mk >> 4) & 0xF)];
        const u32x2 b0 = t2[(mk >> 8) & 0xF], b1 = t2[16 + ((mk >> 12) & 0xF)];
        const u32x4 s0 = u32x4{a0.x, a0.y, a1.x, a1.y};
        const u32x4 s1 = u32x4{b0.x, b0.y, b1.x, b1.y};
        uint32_t w[8];
        w[0] = __builtin_amdgcn_perm(v.y, v.x, s0.x);
        w[1] = __builtin_amdgcn_perm(v.y, v.x, s0.y);
        w[2] = __builtin_amdgcn_perm(v.y, v.x, s0.z);
        w[3] = __builtin_amdgcn_perm(v.y, v.x, s0.w);
        w[4] = __builtin_amdgcn_perm(v.w, v.z, s1.x);
        w[5] = __builtin_amdgcn_perm(v.w, v.z, s1.y);
        w[6] = __builtin_amdgcn_perm(v.w, v.z, s1.z);
        w[7] = __builtin_amdgcn_perm(v.w, v.z, s1.w);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x4 xa = xs[b * bstride + xslot];
            const u32x4 xb = xs[b * bstride + xslot + 32];
            float a = acc[b];
            a = dot2<DT>(w[0], xa.x, a);
            a = dot2<DT>(w[1], xa.y, a);
            a = dot2<DT>(w[2], xa.z, a);
            a = dot2<DT>(w[3], xa.w, a);
            a = dot2<DT>(w[4], xb.x, a);
            a = dot2<DT>(w[5], xb.y, a);
            a = dot2<DT>(w[6], xb.z, a);
            a = dot2<DT>(w[7], xb.w, a);
            acc[b] = a;
        }
    }
}

// Up to kMaxParts matrices with the same K (and format) multiplied by the
// same x in one launch, their rows concatenated: part p owns rows
// [begin[p], begin[p+1]) of the launch.  A single matrix is one part.
// Gated mode (glu = 1) takes two parts of begin[1] rows each, the gate
// (part 0) and up (part 1) projections of a gated MLP, and writes one output
// h = SiLU(gate x) * (up x) to y[0]; its launch rows interleave the parts
// (row 2i = gate row i, row 2i + 1 = up row i) so that both rows of an output
// are always reduced by one block.  (kMaxParts is one of the argument rules.)

// A part may also scatter its rows into a larger y: with ymap[p] set, its row
// i goes to y row ymap[p][i] of a y whose batch stride is ystride[p] (the
// hybrid format's sparse and dense rows); map entries are clamped into
// [0, ystride), so a bad map can never write outside y.
struct Parts {
    const u32x4* w[kMaxParts];
    const uint16_t* m[kMaxParts];
    uint16_t* y[kMaxParts];
    const int32_t* ymap[kMaxParts];
    int ystride[kMaxParts];
    int begin[kMaxParts + 1];
    int count;
    int glu;
};

__device__ __forceinline__ int mapped_row(const int32_t* ymap, int stride, int rl)
{
    return ymap ? min(max(ymap[rl], 0), stride - 1) : rl;
}

struct RowRef {
    const u32x4* w;      // the row's chunks
    const uint16_t* m;   // the row's mask words (sparse)
    uint16_t* y;         // y[0][row] of its part; batch b at y + b * R
    int R;               // rows of its part
};

// Launch row r (wave-uniform; see Parts for the gated interleave).  The part
// holding r is chosen by selects over the part table, never by an indexed
// read of the kernel arguments.  Only a part with an output-row map reads
// memory here (its map entry).
__device__ __forceinline__ RowRef row_ref(const Parts& P, int r, int C)
{
    RowRef o;
    if (P.glu) {
        const int i = r >> 1;
        const bool up = (r & 1) != 0;
        o.w = (up ? P.w[1] : P.w[0]) + (size_t)i * C;
        o.m = (up ? P.m[1] : P.m[0]) + (size_t)i * C;
        o.y = P.y[0] + i;
        o.R = P.begin[1];
        return o;
    }
    // Parts are in increasing row order, so the last boundary passed names the part.
    const bool p1 = 1 < P.count && r >= P.begin[1];
    const bool p2 = 2 < P.count && r >= P.begin[2];
    const bool p3 = 3 < P.count && r >= P.begin[3];
    const u32x4* w = p3 ? P.w[3] : p2 ? P.w[2] : p1 ? P.w[1] : P.w[0];
    const uint16_t* m = p3 ? P.m[3] : p2 ? P.m[2] : p1 ? P.m[1] : P.m[0];
    uint16_t* y = p3 ? P.y[3] : p2 ? P.y[2] : p1 ? P.y[1] : P.y[0];
    const int32_t* ymap = p3 ? P.ymap[3] : p2 ? P.ymap[2] : p1 ? P.ymap[1] : P.ymap[0];
    const int b0 = p3 ? P.begin[3] : p2 ? P.begin[2] : p1 ? P.begin[1] : 0;
    const int b1 = p3 ? P.begin[4] : p2 ? P.begin[3] : p1 ? P.begin[2] : P.begin[1];
    const int rl = r - b0;
    o.w = w + (size_t)rl * C;
    o.m = m + (size_t)rl * C;
    if (ymap) {
        const int stride = p3 ? P.ystride[3] : p2 ? P.ystride[2] : p1 ? P.ystride[1] : P.ystride[0];
        o.R = stride;
        o.y = y + mapped_row(ymap, stride, rl);
    } else {
        o.R = b1 - b0;
        o.y = y + rl;
    }
    return o;
}

// Weight pointers of launch row r for a row index that differs across lanes:
// the part is chosen by selects over the (wave-uniform) part table, never by
// a dynamic index (which would become a memory load).  y is left unset.
__device__ __forceinline__ RowRef row_ref_lane(const Parts& P, int r, int C)
{
    const int rr = P.glu ? (r >> 1) : r;
    int p = P.glu ? (r & 1) : 0;
    if (!P.glu) {
#pragma unroll
        for (int k = 1; k < kMaxParts; ++k)
            p = (k < P.count && r >= P.begin[k]) ? k : p;
    }
    const u32x4* w = P.w[0];
    const uint16_t* m = P.m[0];
#pragma unroll
    for (int k = 1; k < kMaxParts; ++k) {
        const bool on = p == k;
        w = on ? P.w[k] : w;
        m = on ? P.m[k] : m;
    }
    const int b0 = P.glu ? 0 : (p == 0 ? 0 : p == 1 ? P.begin[1] : p == 2 ? P.begin[2] : P.begin[3]);
    const int rl = P.glu ? rr : r - b0;
    RowRef o;                                    // only the weight pointers are used in the lane layout
    o.w = w + (size_t)rl * C;
    o.m = m + (size_t)rl * C;
    o.y = nullptr;
    o.R = 0;
    return o;
}

// The gated-MLP output element: SiLU(g) * u with SiLU(t) = t / (1 + e^-t),
// from the unrounded fp32 sums.  It is evaluated in double (once per output
// row, so the cost is nil): in fp32, e^-g overflows for g < -88.7 and SiLU
// would flush to 0 where bf16 still holds SiLU(g) * u.  The double result is
// rounded to fp32 and then to the output format, nearest even each time.
template <int DT>
__device__ __forceinline__ uint16_t glu_out(float g, float u)
{
    const double gd = g;
    return from_f32<DT>((float)(gd / (1.0 + exp(-gd)) * (double)u));
}

// Loads chunks [c0 + lane + 64 u] (u < U) of a row.  Every lane issues all U
// loads -- lanes past cend reload chunk 0, and the consumer zeroes them with
// chunk_live() -- so the code is branch-free and the compiler can wait for
// exactly the loads each use needs (loads retire in issue order).
// The row pointers are cast to the global address space so that the loads
// are global (not flat) loads whatever the compiler can prove about where
// the pointers came from.
typedef __attribute__((address_space(1))) const u32x4 gu32x4_t;
typedef __attribute__((address_space(1))) const uint16_t gu16_t;

template <int F, int U>
__device__ __forceinline__ void load_chunks(const u32x4* __restrict__ wrow, const uint16_t* __restrict__ mrow,
                                            int c0, int cend, int lane, u32x4* v, uint32_t* mk)
{
    gu32x4_t* gw = (gu32x4_t*)wrow;
    gu16_t* gm = (gu16_t*)mrow;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + u * kWave;
        const int cc = c < cend ? c : 0;
        v[u] = __builtin_nontemporal_load(gw + cc);
        if constexpr (F != kDense)
            mk[u] = __builtin_nontemporal_load(gm + cc);
        else
            mk[u] = 0;
    }
}

// Zeroes a chunk loaded by a lane that had no chunk (values and mask), so it
// contributes exactly 0 whatever was reloaded.
__device__ __forceinline__ void chunk_live(bool live, u32x4& v, uint32_t& mk)
{
    v.x = live ? v.x : 0u;
    v.y = live ? v.y : 0u;
    v.z = live ? v.z : 0u;
    v.w = live ? v.w : 0u;
    mk = live ? mk : 0u;
}

// Two rows' chunks at the same columns (a wave holding a pair of rows):
// acc[b] += (va . x[b]) and acc2[b] += (vb . x[b]), each x unit read from LDS
// once for both rows.  Sparse formats only.
template <int F, int DT, int NB>
__device__ __forceinline__ void chunk_dot_pair(const u32x4 va, const uint32_t ma, const u32x4 vb, const uint32_t mb,
                                               const u32x4* __restrict__ tab, const u32x4* __restrict__ xs,
                                               const int xslot, const int bstride, float* acc, float* acc2)
{
    static_assert(F != kDense, "row pairs are a sparse-format plan");
    if constexpr (F == kNM24) {
        const uint32_t* t = reinterpret_cast<const uint32_t*>(tab);
        const uint32_t s0 = t[ma & 0xF], s1 = t[(ma >> 4) & 0xF], s2 = t[(ma >> 8) & 0xF], s3 = t[(ma >> 12) & 0xF];
        const uint32_t q0 = t[mb & 0xF], q1 = t[(mb >> 4) & 0xF], q2 = t[(mb >> 8) & 0xF], q3 = t[(mb >> 12) & 0xF];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x4 xa = xs[b * bstride + xslot];
            const u32x4 xb = xs[b * bstride + xslot + 32];
            float a = acc[b], c = acc2[b];
            a = dot2<DT>(va.x, __builtin_amdgcn_perm(xa.y, xa.x, s0), a);
            c = dot2<DT>(vb.x, __builtin_amdgcn_perm(xa.y, xa.x, q0), c);
            a = dot2<DT>(va.y, __builtin_amdgcn_perm(xa.w, xa.z, s1), a);
            c = dot2<DT>(vb.y, __builtin_amdgcn_perm(xa.w, xa.z, q1), c);
            a = dot2<DT>(va.z, __builtin_amdgcn_perm(xb.y, xb.x, s2), a);
            c = dot2<DT>(vb.z, __builtin_amdgcn_perm(xb.y, xb.x, q2), c);
            a = dot2<DT>(va.w, __builtin_amdgcn_perm(xb.w, xb.z, s3), a);
            c = dot2<DT>(vb.w, __builtin_amdgcn_perm(xb.w, xb.z, q3), c);
            acc[b] = a;
            acc2[b] = c;
        }
    } else {
        const u32x2* t2 = reinterpret_cast<const u32x2*>(tab);
        uint32_t w[8], u[8];
        {
            const u32x4 s0 = u32x4{t2[ma & 0xF].x, t2[ma & 0xF].y, t2[16 + ((ma >> 4) & 0xF)].x,
                                   t2[16 + ((ma >> 4) & 0xF)].y};
            const u32x4 s1 = u32x4{t2[(ma >> 8) & 0xF].x, t2[(ma >> 8) & 0xF].y, t2[16 + ((ma >> 12) & 0xF)].x,
                                   t2[16 + ((ma >> 12) & 0xF)].y};
            w[0] = __builtin_amdgcn_perm(va.y, va.x, s0.x);
            w[1] = __builtin_amdgcn_perm(va.y, va.x, s0.y);
            w[2] = __builtin_amdgcn_perm(va.y, va.x, s0.z);
            w[3] = __builtin_amdgcn_perm(va.y, va.x, s0.w);
            w[4] = __builtin_amdgcn_perm(va.w, va.z, s1.x);
            w[5] = __builtin_amdgcn_perm(va.w, va.z, s1.y);
            w[6] = __builtin_amdgcn_perm(va.w, va.z, s1.z);
            w[7] = __builtin_amdgcn_perm(va.w, va.z, s1.w);
        }
        {
            const u32x4 s0 = u32x4{t2[mb & 0xF].x, t2[mb & 0xF].y, t2[16 + ((mb >> 4) & 0xF)].x,
                                   t2[16 + ((mb >> 4) & 0xF)].y};
            const u32x4 s1 = u32x4{t2[(mb >> 8) & 0xF].x, t2[(mb >> 8) & 0xF].y, t2[16 + ((mb >> 12) & 0xF)].x,
                                   t2[16 + ((mb >> 12) & 0xF)].y};
            u[0] = __builtin_amdgcn_perm(vb.y, vb.x, s0.x);
            u[1] = __builtin_amdgcn_perm(vb.y, vb.x, s0.y);
            u[2] = __builtin_amdgcn_perm(vb.y, vb.x, s0.z);
            u[3] = __builtin_amdgcn_perm(vb.y, vb.x, s0.w);
            u[4] = __builtin_amdgcn_perm(vb.w, vb.z, s1.x);
            u[5] = __builtin_amdgcn_perm(vb.w, vb.z, s1.y);
            u[6] = __builtin_amdgcn_perm(vb.w, vb.z, s1.z);
            u[7] = __builtin_amdgcn_perm(vb.w, vb.z, s1.w);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x4 xa = xs[b * bstride + xslot];
            const u32x4 xb = xs[b * bstride + xslot + 32];
            const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            float a = acc[b], c = acc2[b];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                a = dot2<DT>(w[k], xv[k], a);
                c = dot2<DT>(u[k], xv[k], c);
            }
            acc[b] = a;
            acc2[b] = c;
        }
    }
}

// ---- row-slice kernel ------------------------------------------------------

// A block holds rows_per_block rows x S = 2^ls K-slices, one wave per (row,
// slice).  A wave issues its share of the block's x loads -- one 16-byte
// unit per thread into a register when that covers x (xreg), else
// global-to-LDS loads, which hold no registers -- and then all of its chunk
// loads (at most CPL), builds the selector table, waits for its own x loads
// (storing a register unit), meets the block, computes chunk by chunk as the
// weights land, reduces across lanes, and a row's S slice sums are added in
// slice order.  With xfirst, every wave of the block issues its x loads
// before any wave issues weight loads (an issue-order barrier; nothing is
// waited for): a CU serves its loads roughly in issue order, and a block
// cannot compute until all of its x is in LDS, so x queued behind the
// block's own weights would hold every wave of the block until nearly all of
// its data had arrived.
// The body takes its block index as an argument so that one launch can run
// two plans side by side (hybrid_rowslice_kernel).
//
// RPW = 2 (sparse rows, S = 1): each wave holds two consecutive rows (a
// gated launch's gate and up rows of one output), loads both rows' chunks,
// and multiplies them against the same x reads; the block's rows_per_block
// rows are then two per wave, so a block's x and its per-wave work serve
// twice the rows.
template <int F, int DT, int NB, int CPL, int XU, int RPW = 1>
__device__ __forceinline__ void rowslice_body(const Parts& P, const u32x4* __restrict__ x4, int R, int K, int ls,
                                              int rows_per_block, int xfirst, int xreg, unsigned blk)
{
    static_assert(RPW == 1 || (RPW == 2 && F != kDense), "row pairs: sparse formats");
    extern __shared__ u32x4 smem[];
    constexpr int COLS = chunk_cols<F>();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nwaves = blockDim.x / kWave;
    const int S = 1 << ls;
    const int lr = wave >> ls, sl = wave & (S - 1);
    const int r = blk * rows_per_block + lr * RPW;
    const bool active = r < R;
    const bool active2 = RPW == 2 && r + 1 < R;
    const int C = (int)((unsigned)K / COLS);
    // Slices start on 32-chunk boundaries, so that a lane's x slots are one
    // base plus a fixed step per load slot (the last slice may be shorter).
    const int cps = (((C + S - 1) >> ls) + 31) & ~31;
    const int cbeg = sl * cps, cend = active ? min(C, cbeg + cps) : cbeg;
    const RowRef row = row_ref(P, active ? r : 0, C);
    const RowRef row2 = row_ref(P, active2 ? r + 1 : 0, C);   // (RPW = 2; its rows stay in [cbeg, cend))

    u32x4* tab = smem;
    u32x4* xs = smem + table_units<F>();
    const int bstride = x_row_units(K);
    float* part = reinterpret_cast<float*>(xs + NB * bstride);
    const int xunits = NB * (K >> 3);
    u32x4 xr[XU];
    if (xreg) {                                  // XU x units per thread cover x
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int i = threadIdx.x + u * blockDim.x;
            xr[u] = x4[i < xunits ? i : 0];
        }
    } else {
        x_dma<F, NB>(x4, K, bstride, lds_offset_of(xs), wave, nwaves, lane);
    }
    if (xfirst)
        __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    u32x4 v[CPL], v2[RPW == 2 ? CPL : 1];
    uint32_t mk[CPL], mk2[RPW == 2 ? CPL : 1];
    load_chunks<F, CPL>(row.w, row.m, cbeg, cend, lane, v, mk);
    if constexpr (RPW == 2)
        load_chunks<F, CPL>(row2.w, row2.m, cbeg, cend, lane, v2, mk2);
    build_table<F>(tab);
    constexpr int NW = (F == kDense ? CPL : 2 * CPL) * RPW;   // weight loads issued after x
    if (xreg) {
        wait_vmcnt<NW>();
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int i = threadIdx.x + u * blockDim.x;
            if (i < xunits) {
                const int b = NB == 1 ? 0 : i / (K >> 3);
                xs[x_slot<F>(b, i - b * (K >> 3), bstride)] = xr[u];
            }
        }
    }
    // This wave's x loads, issued before its weight loads, have landed and its
    // LDS stores are done; then the block meets at a barrier with no memory
    // fence (a fence would wait for the weight loads too).
    wait_vmcnt_lgkm0<NW>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    float acc[NB], acc2[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        acc[b] = 0.f;
        acc2[b] = 0.f;
    }
    const int xl = chunk_xslot<F>(cbeg + lane);      // cbeg % 32 == 0: slot u is xl + u * step
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
        if (u * kWave >= cend - cbeg)          // wave-uniform: nothing left in this slot for any lane
            break;
        if ((u + 1) * kWave <= cend - cbeg) {  // wave-uniform: every lane holds a chunk
            if constexpr (RPW == 2)
                chunk_dot_pair<F, DT, NB>(v[u], mk[u], v2[u], mk2[u], tab, xs, xl + u * xslot_step<F>(), bstride, acc,
                                          acc2);
            else
                chunk_dot<F, DT, NB>(v[u], mk[u], tab, xs, xl + u * xslot_step<F>(), bstride, acc);
        } else {
            const bool live = cbeg + lane + u * kWave < cend;
            chunk_live(live, v[u], mk[u]);
            if constexpr (RPW == 2) {
                chunk_live(live, v2[u], mk2[u]);
                chunk_dot_pair<F, DT, NB>(v[u], mk[u], v2[u], mk2[u], tab, xs, live ? xl + u * xslot_step<F>() : 0,
                                          bstride, acc, acc2);
            } else {
                chunk_dot<F, DT, NB>(v[u], mk[u], tab, xs, live ? xl + u * xslot_step<F>() : 0, bstride, acc);
            }
        }
    }
    float sum[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        sum[b] = wave_sum(acc[b]);
    if constexpr (RPW == 2) {
        // S = 1: the pair's sums go straight to y (gated: rows r and r + 1 are
        // the gate and up rows of one output).
        float sum2[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            sum2[b] = wave_sum(acc2[b]);
        if (lane != 0)
            return;
        if (P.glu) {
            if (active)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    row.y[(size_t)b * row.R] = glu_out<DT>(sum[b], sum2[b]);
            return;
        }
        if (active)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                row.y[(size_t)b * row.R] = from_f32<DT>(sum[b]);
        if (active2)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                row2.y[(size_t)b * row2.R] = from_f32<DT>(sum2[b]);
        return;
    }
    if (S == 1 && !P.glu) {
        if (active && lane == 0)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                row.y[(size_t)b * row.R] = from_f32<DT>(sum[b]);
        return;
    }
    if (lane == 0)
#pragma unroll
        for (int b = 0; b < NB; ++b)
            part[wave * NB + b] = sum[b];
    __syncthreads();
    if (P.glu) {
        // Local rows lr (gate, even) and lr + 1 (up) hold one output row; the
        // gate row's first slice combines both, each in slice order.
        if (active && (lr & 1) == 0 && sl == 0 && lane == 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float g = part[wave * NB + b], u = part[(wave + S) * NB + b];
                for (int j = 1; j < S; ++j) {
                    g += part[(wave + j) * NB + b];
                    u += part[(wave + S + j) * NB + b];
                }
                row.y[(size_t)b * row.R] = glu_out<DT>(g, u);
            }
        }
        return;
    }
    if (active && sl == 0 && lane == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t = part[wave * NB + b];
            for (int j = 1; j < S; ++j)
                t += part[(wave + j) * NB + b];
            row.y[(size_t)b * row.R] = from_f32<DT>(t);
        }
    }
}

template <int F, int DT, int NB, int CPL, int XU, int RPW = 1>
__global__ __launch_bounds__(1024) void rowslice_kernel(const Parts P, const u32x4* __restrict__ x4, int R, int K,
                                                        int ls, int rows_per_block, int xfirst, int xreg)
{
    rowslice_body<F, DT, NB, CPL, XU, RPW>(P, x4, R, K, ls, rows_per_block, xfirst, xreg, blockIdx.x);
}

// A hybrid matrix (sparse rows PS plus dense rows PD, both scattered into one
// y) in a single launch, so the dense rows do not pay a launch's start-up and
// drain of their own: blocks [0, sparse_blocks) run the sparse rows' row-slice
// plan, the rest the dense rows' plan with twice the slices and half the rows
// per block -- a dense row has twice the chunks of a sparse one at the same
// K, so both plans give a lane the same CPL chunks and a block the same
// waves.
template <int F, int DT, int NB, int CPL, int XU>
__global__ __launch_bounds__(1024) void hybrid_rowslice_kernel(const Parts PS, const Parts PD,
                                                               const u32x4* __restrict__ x4, int RS, int RD, int K,
                                                               int ls, int rows_per_block, int xfirst, int xreg,
                                                               int sparse_blocks)
{
    const unsigned blk = blockIdx.x;
    if (blk < (unsigned)sparse_blocks)
        rowslice_body<F, DT, NB, CPL, XU>(PS, x4, RS, K, ls, rows_per_block, xfirst, xreg, blk);
    else
        rowslice_body<kDense, DT, NB, CPL, XU>(PD, x4, RD, K, ls + 1, rows_per_block / 2, xfirst, xreg,
                                               blk - sparse_blocks);
}

// ---- streaming kernel --------------------------------------------------------

// Wave g of G handles rows g, g + G, g + 2G, ..., so at any moment the grid
// reads one compact band of rows (DRAM-page friendly).  A row is cut into
// groups of U chunks per lane; the wave walks its (row, group) sequence with
// the next group's loads in flight while it multiplies the current one (two
// register buffers).  x is staged in LDS in tiles of tile_cols columns; with
// one tile a row's sum goes straight to y, with several the wave keeps each
// of its rows' partial sums in LDS between tiles (slot = wave * rpw + t).
template <int F, int DT, int NB, int U>
__global__ __launch_bounds__(1024) void stream_kernel(const Parts P, const u32x4* __restrict__ x4, int R, int K,
                                                      int tile_cols)
{
    extern __shared__ u32x4 smem[];
    constexpr int COLS = chunk_cols<F>();
    const int lane = threadIdx.x & (kWave - 1);
    const int nw = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = blockIdx.x * nw + wave;
    const int G = gridDim.x * nw;
    const int C = K / COLS;
    // The wave's t-th row is launch row g + t G; in gated mode it is the gate
    // (t even) or up (t odd) row of output row g + (t / 2) G, so both rows of
    // an output pass through the same wave, one after the other.
    const int per = P.glu ? 2 : 1;
    const int Ru = R / per;                                // rows (outputs) dealt to the waves
    const int rpw = per * ((Ru + G - 1) / G);              // rows per wave, at most
    const int nrows = per * (g < Ru ? (Ru - g + G - 1) / G : 0);
    auto lrow = [&](int t) { return P.glu ? 2 * (g + (t >> 1) * G) + (t & 1) : g + t * G; };
    const bool multi = tile_cols < K;
    float gs[NB];                                          // gated mode, one tile: the gate row's sums
#pragma unroll
    for (int b = 0; b < NB; ++b)
        gs[b] = 0.f;
    const int bstride = x_row_units(tile_cols);

    u32x4* tab = smem;
    u32x4* xs = smem + table_units<F>();
    float* part = reinterpret_cast<float*>(xs + NB * bstride);
    build_table<F>(tab);
    if (multi)
        for (int i = threadIdx.x; i < nw * rpw * NB; i += blockDim.x)
            part[i] = 0.f;

    for (int t0 = 0; t0 < K; t0 += tile_cols) {
        const int tc = min(tile_cols, K - t0);
        const int cb = t0 / COLS, ce = (t0 + tc) / COLS;
        const int gpr = (ce - cb + kWave * U - 1) / (kWave * U);   // groups per row in this tile
        const int ng = nrows * gpr;
        // This tile's x is fetched before its first weight loads are issued:
        // loads retire in issue order, so x fetched behind HBM weight loads
        // would hold every wave at the barrier for a full HBM round trip.
        u32x4 xr[kXU];
        x_fetch_tile<NB>(x4, K, t0, tc, xr);
        u32x4 va[U], vb[U];
        uint32_t ma[U], mb[U];
        {
            const RowRef row = row_ref(P, ng > 0 ? lrow(0) : 0, C);
            load_chunks<F, U>(row.w, row.m, cb, ng > 0 ? ce : cb, lane, va, ma);
        }
        __syncthreads();                          // the previous tile's x is no longer read
        x_store_tile<F, NB>(xs, x4, K, t0, tc, bstride, xr);
        __syncthreads();

        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            acc[b] = 0.f;
        auto consume = [&](int j, const u32x4* v, const uint32_t* mk) {
            const int t = j / gpr, q = j - t * gpr;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // Slots past the row's end for the whole wave are skipped
                // (a wave-uniform branch); a partly filled slot is zeroed.
                if (q * kWave * U + u * kWave >= ce - cb)
                    break;
                const int c = cb + q * kWave * U + lane + u * kWave;
                const bool live = c < ce;
                u32x4 vv = v[u];
                uint32_t mm = mk[u];
                chunk_live(live, vv, mm);
                chunk_dot<F, DT, NB>(vv, mm, tab, xs, live ? chunk_xslot<F>(c - cb) : 0, bstride, acc);
            }
            if (q == gpr - 1) {
                const RowRef row = row_ref(P, lrow(t), C);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float sum = wave_sum(acc[b]);
                    if (lane == 0) {
                        if (multi)
                            part[(wave * rpw + t) * NB + b] += sum;
                        else if (!P.glu)
                            row.y[(size_t)b * row.R] = from_f32<DT>(sum);
                        else if (t & 1)
                            row.y[(size_t)b * row.R] = glu_out<DT>(gs[b], sum);
                    }
                    gs[b] = sum;
                    acc[b] = 0.f;
                }
            }
        };
        auto fetch = [&](int j, u32x4* v, uint32_t* mk) {
            const int t = j / gpr, q = j - t * gpr;
            const RowRef row = row_ref(P, lrow(t), C);
            load_chunks<F, U>(row.w, row.m, cb + q * kWave * U, ce, lane, v, mk);
        };
        for (int j = 0; j < ng; j += 2) {
            if (j + 1 < ng)
                fetch(j + 1, vb, mb);
            consume(j, va, ma);
            if (j + 1 < ng) {
                if (j + 2 < ng)
                    fetch(j + 2, va, ma);
                consume(j + 1, vb, mb);
            }
        }
    }
    if (multi && lane == 0) {
        // part[] of this wave was written only by this wave's lane 0: no barrier needed.
        for (int t = 0; t < nrows; ++t) {
            const RowRef row = row_ref(P, lrow(t), C);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (!P.glu)
                    row.y[(size_t)b * row.R] = from_f32<DT>(part[(wave * rpw + t) * NB + b]);
                else if (t & 1)
                    row.y[(size_t)b * row.R] =
                        glu_out<DT>(part[(wave * rpw + t - 1) * NB + b], part[(wave * rpw + t) * NB + b]);
            }
        }
    }
}

// ---- matrix-core kernel for batched products ----------------------------------

// With several activation vectors the VALU kernels above pay one byte-permute
// and one dot2 per group per vector, plus the LDS reads of every vector's x;
// from B ~ 6 that, not HBM, sets their pace.  Here the matrix cores take the
// batch: a wave multiplies a 16-row tile of W by x^T (16 batch columns per
// tile of the batch) with v_mfma_f32_16x16x32 over one K-slice.  In the
// operand layout lane l (i = l % 16, quarter q = l / 16) holds chunk
// c0 + 4 t + q of tile row i at step t; each chunk's 16 (dense: 8) columns are
// COLS / 4 k-blocks of 4 columns, and the weights of a k-block -- 4 dense
// weights of one row -- are rebuilt from the packed values with two byte
// permutes (2:4: one group; 4:8: half a group; dense: a copy).  A matrix-core
// step takes two k-blocks (8 columns of the chunk) per lane as its A operand
// and the same 8 columns of x row i, one staged 16-byte unit, as its B
// operand; lanes of batch rows past B repeat row B - 1 and their outputs are
// dropped.  gfx950's K = 32 form runs at twice the rate of the 16x16x16 one;
// only the pairing of A's and B's k-values matters, and both take the lane's
// 8 halves in column order.  The matrix core reduces over k, so no
// cross-lane reduction is needed: the slices of a tile add up in LDS in slice
// order.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

template <int DT>
__device__ __forceinline__ f32x4 mfma16k32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (DT == NM_FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8v, a), __builtin_bit_cast(f16x8v, b), c, 0,
                                                      0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c,
                                                       0, 0, 0);
}

// 2:4.  Nibble n marks the kept columns j0 < j1 of a 4-column group; the two
// selectors (dense dword 0 = columns 0, 1; dword 1 = columns 2, 3) move the
// group's first stored value (bytes 0, 1 of its dword) to column j0, the
// second (bytes 2, 3) to j1, and zero bytes (0x0C) elsewhere.  Nibbles
// without exactly two bits give zeros.
__device__ u32x2 expand24(uint32_t n)
{
    uint32_t sel[2] = {0x0C0C0C0Cu, 0x0C0C0C0Cu};
    if (__builtin_popcount(n) == 2) {
        const uint32_t js[2] = {(uint32_t)__builtin_ctz(n), 31u - (uint32_t)__builtin_clz(n)};
        for (uint32_t k = 0; k < 2; ++k) {
            const uint32_t p = js[k], shift = 16 * (p & 1);
            sel[p >> 1] = (sel[p >> 1] & ~(0xFFFFu << shift)) | (((2 * k) | ((2 * k + 1) << 8)) << shift);
        }
    }
    return u32x2{sel[0], sel[1]};
}


template <int F>
__device__ __forceinline__ void build_mfma_table(u32x4* tab)
{
    if constexpr (F == kNM24) {
        u32x2* t2 = reinterpret_cast<u32x2*>(tab);
        for (unsigned t = threadIdx.x; t < 16; t += blockDim.x)
            t2[t] = expand24(t);
    } else if constexpr (F == kNM48) {
        // the VALU kernels' nibble tables: entries 0-15 low nibbles, 16-31 high
        u32x2* t2 = reinterpret_cast<u32x2*>(tab);
        for (unsigned t = threadIdx.x; t < 32; t += blockDim.x)
            t2[t] = t < 16 ? select48_nibble(t, 0) : select48_nibble(t - 16, 4u - __builtin_popcount(t - 16));
    }
}


// Loading in the operand layout would stream each row in 64-byte pieces (one
// per lane quarter): a load instruction would touch 16 rows, and the per-CU
// limit on outstanding cache-line requests, not HBM, would set the pace
// (measured: ~2 TB/s).  So a wave loads its 16-row tile in stages of 16 chunks per row:
// each load instruction reads 256 contiguous bytes of four rows (full lines),
// the stage goes to a wave-private LDS buffer, and the matrix-core operands
// are read back from there.  The next stage's loads are in flight while the
// current one is multiplied; x for a stage is fetched from L2 just before the
// next stage's weight loads, so it never waits behind them.  Each lane's row
// pointers are formed once, by selects over the parts (an index into the
// kernel arguments that varies by lane would become a memory load).

template <int F, int DT, int NT>
__global__ __launch_bounds__(512) void mfma_stage_kernel(const Parts P, const u32x4* __restrict__ x4, int R, int K,
                                                         int B, int S, int tiles_per_block)
{
    extern __shared__ u32x4 smem[];
    constexpr int COLS = chunk_cols<F>();
    constexpr int XC = COLS / 8;                 // 16-byte x units per chunk
    constexpr int KB = COLS / 4;                 // k-blocks per chunk
    constexpr int T = kStageChunks / 4;          // matrix-core steps per stage
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lt = wave / S, sl = wave - lt * S;
    const int r0 = (blockIdx.x * tiles_per_block + lt) * 16;
    const int C = K / COLS;
    const int cps = ((C + S - 1) / S + kStageChunks - 1) / kStageChunks * kStageChunks;
    const int cbeg = min(C, sl * cps), cend = min(C, cbeg + cps);
    const int nst = r0 < R ? (cend - cbeg + kStageChunks - 1) / kStageChunks : 0;
    const int i = lane & 15, q = lane >> 4;      // matrix-core layout
    constexpr int RPL = kWave / kStageChunks;    // rows per load instruction
    constexpr int NL = 16 / RPL;                 // load instructions per stage
    const int lrow = lane / kStageChunks, lc = lane % kStageChunks;  // load layout: row RPL rr + lrow, chunk c0 + lc
    const u32x4* xrow[NT];                       // the lane's x row (B K / 8 units can pass 2^31)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        xrow[nt] = x4 + (size_t)min(16 * nt + i, B - 1) * (K / 8);
    const u32x4* wp[NL];
    const uint16_t* mp[NL];
#pragma unroll
    for (int rr = 0; rr < NL; ++rr) {
        const RowRef row = row_ref_lane(P, min(r0 + RPL * rr + lrow, R - 1), C);
        wp[rr] = row.w;
        mp[rr] = row.m;
    }
    const u32x4* tab = smem;
    uint8_t* stage = reinterpret_cast<uint8_t*>(smem + mfma_table_units<F>()) + (size_t)wave * kStageBytes;
    uint8_t* stage_m = stage + 16 * kStagePitch;

    // Two weight register buffers (the stage being staged and the one after
    // it in flight) and one for a stage's x.
    u32x4 va[NL], vb[NL];
    uint32_t ma[NL], mb[NL];
    u32x4 xv[NT][T][XC];
    auto fetch_w = [&](int c0, u32x4* v, uint32_t* m) {
        const int c = c0 + lc;
        const int cc = c < cend ? c : 0;
#pragma unroll
        for (int rr = 0; rr < NL; ++rr) {
            v[rr] = __builtin_nontemporal_load(wp[rr] + cc);
            if constexpr (F != kDense)
                m[rr] = __builtin_nontemporal_load(mp[rr] + cc);
            else
                m[rr] = 0;
        }
    };
    auto fetch_x = [&](int c0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int c = c0 + 4 * t + q;
            const int cc = c < cend ? c : 0;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int h = 0; h < XC; ++h)
                    xv[nt][t][h] = xrow[nt][cc * XC + h];
        }
    };
    auto stash = [&](const u32x4* v, const uint32_t* m) {
#pragma unroll
        for (int rr = 0; rr < NL; ++rr) {
            const int row = RPL * rr + lrow;
            *reinterpret_cast<u32x4*>(stage + row * kStagePitch + lc * 16) = v[rr];
            if constexpr (F != kDense)                 // chunk 4 t + q at 4 q + t: a lane's four masks adjoin
                *reinterpret_cast<uint16_t*>(stage_m + row * kStageMPitch + ((lc & 3) * 4 + (lc >> 2)) * 2) =
                    (uint16_t)m[rr];
        }
    };
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A stage's LDS reads go out together (the lane's four chunks and, in one
    // 8-byte read, their masks), then the selector reads, then the permutes
    // and matrix-core steps: two LDS round trips per stage, not two per chunk.
    // A chunk past the slice's end multiplies as zeros: its mask is cleared
    // (no selector then picks a value; x is finite) or, dense, its values.
    auto consume = [&](int c0) {
        u32x4 vv[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
            vv[t] = *reinterpret_cast<const u32x4*>(stage + i * kStagePitch + (4 * t + q) * 16);
        uint32_t mk[T] = {};
        if constexpr (F != kDense) {
            const u32x2 mq = *reinterpret_cast<const u32x2*>(stage_m + i * kStageMPitch + q * 8);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t m16 = ((t < 2 ? mq.x : mq.y) >> (16 * (t & 1))) & 0xFFFFu;
                mk[t] = c0 + 4 * t + q < cend ? m16 : 0u;
            }
        } else {
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (c0 + 4 * t + q >= cend)
                    vv[t] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint32_t w[4] = {vv[t].x, vv[t].y, vv[t].z, vv[t].w};
            u32x2 a[KB];
            if constexpr (F == kDense) {
#pragma unroll
                for (int s = 0; s < KB; ++s)
                    a[s] = u32x2{w[2 * s], w[2 * s + 1]};
            } else if constexpr (F == kNM24) {
                const u32x2* t2 = reinterpret_cast<const u32x2*>(tab);
#pragma unroll
                for (int s = 0; s < KB; ++s) {               // k-block s = group s: one nibble, one dword
                    const u32x2 sel = t2[(mk[t] >> (4 * s)) & 0xFu];
                    a[s] = u32x2{__builtin_amdgcn_perm(w[s], w[s], sel.x), __builtin_amdgcn_perm(w[s], w[s], sel.y)};
                }
            } else {
                const u32x2* n2 = reinterpret_cast<const u32x2*>(tab);
#pragma unroll
                for (int g = 0; g < 2; ++g) {                // group g: k-blocks 2 g, 2 g + 1
                    const uint32_t mg = (mk[t] >> (8 * g)) & 0xFFu;
                    const u32x2 lo = n2[mg & 0xFu], hi = n2[16 + (mg >> 4)];
                    a[2 * g] = u32x2{__builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], lo.x),
                                     __builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], lo.y)};
                    a[2 * g + 1] = u32x2{__builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], hi.x),
                                         __builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], hi.y)};
                }
            }
            // Two 4-column k-blocks (8 columns, one x unit) per matrix-core step.
#pragma unroll
            for (int h = 0; h < KB / 2; ++h)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt] = mfma16k32<DT>(u32x4{a[2 * h].x, a[2 * h].y, a[2 * h + 1].x, a[2 * h + 1].y},
                                            xv[nt][t][h], acc[nt]);
        }
    };
    // One pipeline step: multiply stage st (in LDS, its x in registers),
    // stage st + 1 (its weights arrived in `cur`), fetch x of st + 1, then
    // the weights of st + 3 into `cur` (st + 2 is in flight in the other
    // buffer).  Loads past the slice's end read chunk 0 and are never used.
    auto step = [&](int c0, u32x4* cv, uint32_t* cm) {
        __builtin_amdgcn_sched_barrier(0);
        consume(c0);
        __builtin_amdgcn_sched_barrier(0);
        stash(cv, cm);                           // after this stage's LDS reads (in order within the wave)
        fetch_x(c0 + kStageChunks);
        __builtin_amdgcn_sched_barrier(0);
        fetch_w(c0 + 3 * kStageChunks, cv, cm);
    };

    build_mfma_table<F>(smem);
    __syncthreads();
    // Every load inside the loop is unconditional, so the compiler counts
    // outstanding loads exactly (a conditional load makes it wait for all).
    if (nst > 0) {
        fetch_w(cbeg, va, ma);
        stash(va, ma);
        fetch_x(cbeg);
        __builtin_amdgcn_sched_barrier(0);
        fetch_w(cbeg + kStageChunks, va, ma);
        fetch_w(cbeg + 2 * kStageChunks, vb, mb);
        int c0 = cbeg;
        int st = 0;
        for (; st + 2 <= nst; st += 2, c0 += 2 * kStageChunks) {
            step(c0, va, ma);
            step(c0 + kStageChunks, vb, mb);
        }
        if (st < nst)
            consume(c0);
    }

    // Slice sums: D[4 q + v][i] of this wave's tile (row 4 q + v, batch column 16 nt + i).
    float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem + mfma_table_units<F>()) +
                                           (size_t)blockDim.x / kWave * kStageBytes);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv)
            part[((wave * NT + nt) * kWave + lane) * 4 + vv] = acc[nt][vv];
    __syncthreads();
    if (sl != 0 || r0 >= R)
        return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int b = 16 * nt + i;
        if (b >= B)
            continue;
        float sum[4];
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
            float t = part[((wave * NT + nt) * kWave + lane) * 4 + vv];
            for (int j = 1; j < S; ++j)
                t += part[(((wave + j) * NT + nt) * kWave + lane) * 4 + vv];
            sum[vv] = t;
        }
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
            const int r = r0 + 4 * q + vv;
            if (r >= R)
                continue;
            const RowRef o = row_ref(P, r, C);
            if (!P.glu)
                o.y[(size_t)b * o.R] = from_f32<DT>(sum[vv]);
            else if ((vv & 1) == 0)              // rows r (gate) and r + 1 (up) of one output
                o.y[(size_t)b * o.R] = glu_out<DT>(sum[vv], sum[vv + 1]);
        }
    }
}

// ---- matrix-core kernel, LDS ring (batches of up to 16 vectors) ---------------

// The staged kernel above passes every weight byte through registers on its
// way to LDS, which caps a CU at 3 waves and ~2 stages in flight, and its x
// loads queue behind weight loads issued after them.  Here the weights go
// straight from HBM to a two-slot LDS ring per wave (16-byte global-to-LDS
// loads), x goes to registers in the same stage order, and a wave's slice of
// K is short enough that a launch has several waves per SIMD.  Layout of one
// slot (16 rows x 16 chunks of a 16-row tile):
//  * values: four 1 KB blocks of 4 rows x 256 bytes; the lane at position p
//    of row r loads chunk p ^ r, so the 16 rows' copies of a chunk fall in
//    different banks when the operand layout reads them back;
//  * masks: 16 rows x 32 bytes; position p of a row holds mask dword
//    2 (p % 4) + p / 4, so that dwords 0, 2, 4, 6 (chunks 4 t + q, q < 2) and
//    1, 3, 5, 7 (q >= 2) each form one 16-byte read.
// A wave multiplies TW 16-row tiles (rows 16 TW w .. 16 TW w + 16 TW - 1) by
// the same staged x, so each byte of x brought to LDS serves TW tiles; NT
// batch tiles of 16 vectors share each weight operand.
//
// SHX (one K-slice per tile): the block's waves share one staged x.  Each
// wave keeps its two-slot weight ring; x goes to a two-slot ring of the
// block, its load instructions dealt round-robin over the waves.  Per stage
// a wave waits for its own loads, then all meet at a barrier (no memory
// fence: each wave's wait already covers its loads into LDS), so after it
// every piece of the stage's x is in place; only then is the next stage's
// x issued, into the slot whose last reads every wave finished before that
// barrier.  Every wave runs all stages (tiles past R read clamped rows and
// store nothing), so the barrier counts match.
//
// KSPLIT (with SHX): the block's waves take one of KS contiguous ranges of
// the stages (split ks = blockIdx.x % KS of tile group blockIdx.x / KS), so a
// short matrix fills the GPU while each staged x still serves several
// tiles.  Each wave writes its tiles' partial sums to scratch; the block then
// counts itself in its group's counter, and the block that arrives last adds
// the KS partials of every tile in split order (fixed, so results do not
// depend on which block is last), writes y and resets the counter to zero
// for the next launch.  The partials and the counter are accessed only as
// agent-scope atomics (coherent across the GPU's L2 caches without cache
// write-back or invalidation, which cost tens of microseconds here), and
// each thread waits for its partial stores to complete before the block's
// counter update, so the last block's reads see them.
struct SplitK {
    float* part;         // KS x (tile groups x tiles_per_block x TW x NT) x 256 floats
    unsigned* cnt;       // one counter per tile group, zero between launches
    int ks;              // splits (KS)
    int stages;          // stages per split (the last may have fewer, or none)
};

// CU-major tile map (SHX without KSPLIT; k = 0: block b takes tiles
// b * tiles_per_block ..).  A launch of k * cus blocks whose blocks all fit
// at once puts block b on CU b % cus (the dispatcher deals blocks to the CUs
// in turn), so CU c's share of the tile units, [c T / cus, (c + 1) T / cus),
// is split over its k blocks, block b = c + j cus taking part j.  The map
// covers each unit once whatever the dispatcher does; only the balance
// depends on it.  Waves past their block's count take no tile.
struct TileMap {
    int tiles;           // T: tile units (TW tiles each)
    int cus;
    int k;               // blocks a CU, 0 = plain map
};

template <int F, int DT, int TW, int NT, bool SHX, bool KSPLIT = false>
__global__ __launch_bounds__(512) void mfma_ring_kernel(const Parts P, const u32x4* __restrict__ x4, int R, int K,
                                                        int B, int S, int tiles_per_block, SplitK sk, TileMap tm)
{
    static_assert(!KSPLIT || SHX, "K-split blocks share their staged x");
    extern __shared__ u32x4 smem[];
    constexpr int COLS = chunk_cols<F>();
    constexpr int XC = COLS / 8;                 // 16-byte x units per chunk
    constexpr int KB = COLS / 4;                 // k-blocks per chunk
    constexpr int T = kStageChunks / 4;          // matrix-core steps per stage
    constexpr int NM = F == kDense ? 0 : 2;      // mask load instructions per stage and tile
    constexpr int UPR = ring_x_units<F>();       // x units per batch row per stage
    constexpr int RPX = kWave / UPR;             // batch rows per x load instruction
    constexpr int TAB = mfma_table_units<F>() * 16;
    constexpr int TBYTES = kRingValues + (F == kDense ? 0 : kRingMasks);   // one tile's part of a slot
    constexpr int XOFF = TW * TBYTES;            // x within a wave's slot (without SHX)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lt = wave / S, sl = wave - lt * S;
    const int ks = KSPLIT ? (int)(blockIdx.x % (unsigned)sk.ks) : 0;
    const int grp = KSPLIT ? (int)(blockIdx.x / (unsigned)sk.ks) : (int)blockIdx.x;
    int unit0 = grp * tiles_per_block + lt;
    if (SHX && !KSPLIT && tm.k > 0) {
        const int c = grp % tm.cus, j = grp / tm.cus;
        const int s0 = (int)((int64_t)c * tm.tiles / tm.cus);
        const int n = (int)((int64_t)(c + 1) * tm.tiles / tm.cus) - s0;
        const int f = s0 + j * n / tm.k, l = s0 + (j + 1) * n / tm.k;
        unit0 = f + lt < l ? f + lt : tm.tiles;  // past the block's count: no tile
    }
    const int r0 = (int)min((int64_t)unit0 * 16 * TW, (int64_t)R);
    // SHX: a wave with no rows streams no weights and multiplies nothing, but
    // still loads its share of x and meets the block at every stage.
    const bool idle = SHX && r0 >= R;
    // Slice sl takes stages sl, sl + S, sl + 2 S, ... of the row: the waves
    // of a launch move through K together.
    const int C = K / COLS;
    const int NS = (C + kStageChunks - 1) / kStageChunks;
    // KSPLIT: stages st0 .. st0 + nst - 1 (uniform over the block: the barrier counts match)
    const int st0 = KSPLIT ? ks * sk.stages : 0;
    const int nst = KSPLIT ? max(0, min(sk.stages, NS - st0))
                           : SHX ? NS : (r0 < R && sl < NS) ? (NS - sl + S - 1) / S : 0;
    const int i = lane & 15, q = lane >> 4;      // operand layout: row / batch column i, k-quarter q
    const int nxi = ring_x_rows<F>(B) / RPX;     // x load instructions per stage (1 .. 16)
    const int nwaves = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
    // Without SHX a slot holds the wave's tiles and x; with it, only the tiles.
    const int slot_bytes = SHX ? TW * TBYTES : ring_slot_bytes<F, TW>(B);
    const int xslot_bytes = ring_x_rows<F>(B) * UPR * 16;
    const uint32_t xring = (uint32_t)TAB + (uint32_t)nwaves * 2u * (uint32_t)slot_bytes;   // SHX: the block's x
    constexpr int NW = TW * (4 + NM);            // weight loads per stage

    // Per-lane sources.  Values: tile tw, instruction rr, row 4 rr + lane / 16,
    // chunk (lane % 16) ^ row.  Masks: instruction h, row 8 h + lane / 8, dword
    // 2 (lane % 4) + (lane % 8) / 4.  x: instruction n, batch row
    // n RPX + lane / UPR (past B: row B - 1 again, never read), unit
    // (lane % UPR) ^ (row % 16) of the stage.
    const u32x4* vsrc[TW][4];
    int vchunk[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
        vchunk[rr] = (lane & 15) ^ (4 * rr + (lane >> 4));
    const uint16_t* msrc[TW][2] = {};
    const int mchunk = 2 * (2 * (lane & 3) + ((lane & 7) >> 2));
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            vsrc[tw][rr] = row_ref_lane(P, min(r0 + 16 * tw + 4 * rr + (lane >> 4), R - 1), C).w;
        if constexpr (NM > 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                msrc[tw][h] = row_ref_lane(P, min(r0 + 16 * tw + 8 * h + (lane >> 3), R - 1), C).m;
        }
    }
    const uint32_t ring = (uint32_t)TAB + (uint32_t)wave * 2u * (uint32_t)slot_bytes;
    const uint8_t* ring_p = reinterpret_cast<const uint8_t*>(smem) + ring;

    // Stage st's weights into slot `slot`, and (issue_x) its x; chunks past the
    // row's end load the stage's first chunk instead (in bounds; never
    // multiplied).
    auto issue_w = [&](int st, int slot) {
        if (idle)
            return;
        const int c0 = (sl + (st0 + st) * S) * kStageChunks;
        const uint32_t base = ring + (uint32_t)(slot * slot_bytes);
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int c = c0 + vchunk[rr];
                load_to_lds<16>(vsrc[tw][rr] + (c < C ? c : c0), base + tw * TBYTES + rr * 1024);
            }
            if constexpr (NM > 0) {
                const int c = c0 + mchunk;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    load_to_lds<4>(msrc[tw][h] + (c < C ? c : c0), base + tw * TBYTES + kRingValues + h * 256);
            }
        }
    };
    auto issue_x = [&](int st, int slot) {
        const int c0 = (sl + (st0 + st) * S) * kStageChunks;
        const uint32_t xbase =
            SHX ? xring + (uint32_t)(slot * xslot_bytes) : ring + (uint32_t)(slot * slot_bytes) + (uint32_t)XOFF;
        for (int n = SHX ? wave : 0; n < nxi; n += SHX ? nwaves : 1) {
            const int b = n * RPX + lane / UPR;
            const int u = (lane % UPR) ^ (b & 15);
            const u32x4* xs = x4 + (size_t)min(b, B - 1) * (K / 8) + c0 * XC;
            load_to_lds<16>(xs + (c0 + u / XC < C ? u : u % XC), xbase + n * 1024);
        }
    };

    f32x4 acc[TW][NT];
#pragma unroll
    for (int tw = 0; tw < TW; ++tw)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc[tw][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4* tab = smem;
    int xi[NT];                                  // batch columns past B read row B - 1; results dropped
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        xi[nt] = min(16 * nt + i, B - 1);
    // Multiply stage st from `slot`: the x operands once, then per tile one
    // round of value and mask reads, one of selector reads, the permutes and
    // the matrix-core steps.  A chunk past the row's end multiplies as zeros
    // (mask cleared: no selector picks a value, and x is finite; dense:
    // values cleared).
    auto consume = [&](int st, int slot) {
        const int c0 = (sl + (st0 + st) * S) * kStageChunks;
        const uint8_t* sv0 = ring_p + slot * slot_bytes;
        const uint8_t* sxs = SHX ? reinterpret_cast<const uint8_t*>(smem) + xring + slot * xslot_bytes : sv0 + XOFF;
        u32x4 xx[NT][T][XC];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint8_t* sx = sxs + xi[nt] * (UPR * 16);
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int h = 0; h < XC; ++h)
                    xx[nt][t][h] =
                        *reinterpret_cast<const u32x4*>(sx + ((((4 * t + q) * XC + h) ^ (xi[nt] & 15)) * 16));
        }
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
            const uint8_t* sv = sv0 + tw * TBYTES;
            u32x4 vv[T];
#pragma unroll
            for (int t = 0; t < T; ++t)
                vv[t] = *reinterpret_cast<const u32x4*>(sv + (i >> 2) * 1024 + (i & 3) * 256 + (((4 * t + q) ^ i) * 16));
            uint32_t mk[T] = {};
            if constexpr (F != kDense) {
                const u32x4 md = *reinterpret_cast<const u32x4*>(sv + kRingValues + i * 32 + (q >> 1) * 16);
                const uint32_t mw[4] = {md.x, md.y, md.z, md.w};
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const uint32_t m16 = (mw[t] >> (16 * (q & 1))) & 0xFFFFu;
                    mk[t] = c0 + 4 * t + q < C ? m16 : 0u;
                }
            } else {
#pragma unroll
                for (int t = 0; t < T; ++t)
                    if (c0 + 4 * t + q >= C)
                        vv[t] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t w[4] = {vv[t].x, vv[t].y, vv[t].z, vv[t].w};
                u32x2 a[KB];
                if constexpr (F == kDense) {
#pragma unroll
                    for (int s = 0; s < KB; ++s)
                        a[s] = u32x2{w[2 * s], w[2 * s + 1]};
                } else if constexpr (F == kNM24) {
                    const u32x2* t2 = reinterpret_cast<const u32x2*>(tab);
#pragma unroll
                    for (int s = 0; s < KB; ++s) {
                        const u32x2 sel = t2[(mk[t] >> (4 * s)) & 0xFu];
                        a[s] = u32x2{__builtin_amdgcn_perm(w[s], w[s], sel.x), __builtin_amdgcn_perm(w[s], w[s], sel.y)};
                    }
                } else {
                    const u32x2* n2 = reinterpret_cast<const u32x2*>(tab);
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        const uint32_t mg = (mk[t] >> (8 * g)) & 0xFFu;
                        const u32x2 lo = n2[mg & 0xFu], hi = n2[16 + (mg >> 4)];
                        a[2 * g] = u32x2{__builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], lo.x),
                                         __builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], lo.y)};
                        a[2 * g + 1] = u32x2{__builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], hi.x),
                                             __builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], hi.y)};
                    }
                }
                // Two 4-column k-blocks (8 columns of the chunk, one staged x
                // unit) per matrix-core step.
#pragma unroll
                for (int h = 0; h < KB / 2; ++h)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[tw][nt] = mfma16k32<DT>(u32x4{a[2 * h].x, a[2 * h].y, a[2 * h + 1].x, a[2 * h + 1].y},
                                                    xx[nt][t][h], acc[tw][nt]);
            }
        }
    };

    build_mfma_table<F>(smem);
    __syncthreads();
    // One stage in flight while the previous one is multiplied: issue the
    // weights of st + 1, wait until only those are outstanding (loads complete
    // in order, so st's weights and its x, issued after them, have landed),
    // meet the block (SHX), issue the x of st + 1 (a short L2 read, done during
    // the products of st), multiply st.  The wait counts are fixed; no load in
    // the loop writes registers.
    if (nst > 0) {
        issue_w(0, 0);
        issue_x(0, 0);
        for (int st = 0; st < nst; ++st) {
            const bool more = st + 1 < nst;
            if (more)
                issue_w(st + 1, (st + 1) & 1);
            if (more && !idle)
                wait_vmcnt<NW>();
            else
                wait_vmcnt<0>();                 // (a wave with no rows has only x loads in flight)
            if constexpr (SHX) {                 // every wave's share of the stage's x has landed
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            if (more)
                issue_x(st + 1, (st + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            if (!idle)
                consume(st, st & 1);
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the slot's reads are done before it is refilled
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if constexpr (KSPLIT) {
        // This wave's partial sums: KS x units x TW x NT blocks of 64 lanes x 4 floats.
        const int units = (int)(gridDim.x / (unsigned)sk.ks) * tiles_per_block;
        const int unit = grp * tiles_per_block + lt;
#pragma unroll
        for (int tw = 0; tw < TW; ++tw)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float* dst = sk.part + ((((size_t)ks * units + unit) * TW + tw) * NT + nt) * 256 + lane * 4;
#pragma unroll
                for (int vv = 0; vv < 4; ++vv)
                    __hip_atomic_store(dst + vv, acc[tw][nt][vv], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        wait_vmcnt<0>();                         // this thread's partial stores are complete
        // The flag lives in wave 0's ring, idle once every wave is past its
        // last stage (static LDS would move the offsets the ring loads use).
        int* last_block = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(smem) + TAB);
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(sk.cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *last_block = old == (unsigned)sk.ks - 1u;
        }
        __syncthreads();
        if (!*last_block)
            return;
        if (threadIdx.x == 0)
            __hip_atomic_store(sk.cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r0 >= R)
            return;
#pragma unroll
        for (int tw = 0; tw < TW; ++tw)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int b = 16 * nt + i;
                float sum[4] = {0.f, 0.f, 0.f, 0.f};
                // The partials of up to JB splits are loaded at once (one
                // round trip instead of one per split), then added in split
                // order.
                constexpr int JB = 8;
                for (int j0 = 0; j0 < sk.ks; j0 += JB) {
                    float pv[JB][4];
#pragma unroll
                    for (int jj = 0; jj < JB; ++jj) {
                        const int j = min(j0 + jj, sk.ks - 1);        // past the last split: loaded, not added
                        const float* src = sk.part + ((((size_t)j * units + unit) * TW + tw) * NT + nt) * 256 + lane * 4;
#pragma unroll
                        for (int vv = 0; vv < 4; ++vv)
                            pv[jj][vv] = __hip_atomic_load(src + vv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                    for (int jj = 0; jj < JB; ++jj)
                        if (j0 + jj < sk.ks)
#pragma unroll
                            for (int vv = 0; vv < 4; ++vv)
                                sum[vv] += pv[jj][vv];
                }
                if (b >= B)
                    continue;
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    const int r = r0 + 16 * tw + 4 * q + vv;
                    if (r >= R)
                        continue;
                    const RowRef o = row_ref(P, r, C);
                    if (!P.glu)
                        o.y[(size_t)b * o.R] = from_f32<DT>(sum[vv]);
                    else if ((vv & 1) == 0)      // rows r (gate) and r + 1 (up) of one output
                        o.y[(size_t)b * o.R] = glu_out<DT>(sum[vv], sum[vv + 1]);
                }
            }
        return;
    }

    // Slice sums through the wave's own ring (no loads into it are pending):
    // D[4 q + v][i] of tile tw and batch tile nt (row 16 tw + 4 q + v, batch
    // column 16 nt + i).
    __builtin_amdgcn_s_waitcnt(0xC07F);
    float* part = reinterpret_cast<float*>(smem) + ring / 4;
#pragma unroll
    for (int tw = 0; tw < TW; ++tw)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv)
                part[((tw * NT + nt) * kWave + lane) * 4 + vv] = acc[tw][nt][vv];
    __syncthreads();
    if (sl != 0 || r0 >= R)
        return;
#pragma unroll
    for (int tw = 0; tw < TW; ++tw)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int b = 16 * nt + i;
            if (b >= B)
                continue;
            float sum[4];
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int e = ((tw * NT + nt) * kWave + lane) * 4 + vv;
                float t = part[e];
                for (int j = 1; j < S; ++j)
                    t += part[j * (2 * slot_bytes / 4) + e];
                sum[vv] = t;
            }
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int r = r0 + 16 * tw + 4 * q + vv;
                if (r >= R)
                    continue;
                const RowRef o = row_ref(P, r, C);
                if (!P.glu)
                    o.y[(size_t)b * o.R] = from_f32<DT>(sum[vv]);
                else if ((vv & 1) == 0)          // rows r (gate) and r + 1 (up) of one output
                    o.y[(size_t)b * o.R] = glu_out<DT>(sum[vv], sum[vv + 1]);
            }
        }
}

// ---- generic N:M (any N < M, M in {4, 8}, K % 8 == 0) --------------------------

// One lane step covers one mask byte (8 columns: two 4-groups or one
// 8-group) and its 8 / M * N values at offset q * that (the fixed step).
template <int DT, int NB>
__device__ __forceinline__ void generic_row(const uint16_t* __restrict__ vrow, const uint8_t* __restrict__ mrow,
                                            const uint16_t* __restrict__ x, int K, int N, int M, int lane, float* acc)
{
    const int vpb = 8 / M * N;
#pragma unroll
    for (int b = 0; b < NB; ++b)
        acc[b] = 0.f;
    for (int q = lane; q < K / 8; q += kWave) {
        const uint32_t mb = mrow[q];
        const uint16_t* vp = vrow + (size_t)q * vpb;
        int k = 0;
        for (int j = 0; j < 8; ++j) {
            if (((mb >> j) & 1u) && k < vpb) {
                const float w = to_f32<DT>(vp[k]);
                ++k;
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[b] = fmaf(w, to_f32<DT>(x[(size_t)b * K + 8 * q + j]), acc[b]);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
        acc[b] = wave_sum(acc[b]);
}

// One wave per output row.  With values2 set (gated mode) the wave also
// reduces row `row` of the second matrix and writes SiLU(first) * second.
template <int DT, int NB>
__global__ __launch_bounds__(256) void generic_spmv_kernel(const uint16_t* __restrict__ values,
                                                           const uint8_t* __restrict__ masks,
                                                           const uint16_t* __restrict__ values2,
                                                           const uint8_t* __restrict__ masks2,
                                                           const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                           int R, int K, int N, int M, const int32_t* __restrict__ ymap,
                                                           int ystride)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (row >= R)                                // whole wave leaves together
        return;
    const size_t vrow = (size_t)(K / M) * N;
    float acc[NB];
    generic_row<DT, NB>(values + (size_t)row * vrow, masks + (size_t)row * (K / 8), x, K, N, M, lane, acc);
    const int ys = ymap ? ystride : R;
    const int yr = mapped_row(ymap, ys, row);
    if (values2) {
        float acc2[NB];
        generic_row<DT, NB>(values2 + (size_t)row * vrow, masks2 + (size_t)row * (K / 8), x, K, N, M, lane, acc2);
        if (lane == 0)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                y[(size_t)b * ys + yr] = glu_out<DT>(acc[b], acc2[b]);
        return;
    }
    if (lane == 0)
#pragma unroll
        for (int b = 0; b < NB; ++b)
            y[(size_t)b * ys + yr] = from_f32<DT>(acc[b]);
}

__global__ void fill_zero_kernel(uint16_t* __restrict__ y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        y[i] = 0;
}

// ---- pack ---------------------------------------------------------------------

constexpr uint32_t kStatusBadMask = 1u << 0;
constexpr uint32_t kStatusNaN = 1u << 1;

template <int DT>
__device__ __forceinline__ uint32_t inf_code()
{
    return DT == NM_FP16 ? 0x7C00u : 0x7F80u;
}

// One thread per (row, mask byte) = 8 columns: two 4-groups or one 8-group.
// With rowmap set, output row o packs source row rowmap[o] of W (and keep);
// bpr = K / 8 mask bytes per row.
__device__ __forceinline__ int64_t source_unit(const int32_t* rowmap, int64_t i, int64_t bpr)
{
    return rowmap ? (int64_t)rowmap[i / bpr] * bpr + i % bpr : i;
}

template <int DT>
__global__ __launch_bounds__(256) void pack_check_kernel(const u32x4* __restrict__ W, const uint8_t* __restrict__ keep,
                                                         int64_t nbytes, int N, int M, uint32_t* __restrict__ status,
                                                         const int32_t* __restrict__ rowmap, int64_t bpr)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nbytes)
        return;
    const int64_t u = source_unit(rowmap, i, bpr);
    uint32_t bad = 0;
    if (keep) {
        const uint8_t* kp = keep + 8 * u;
        for (int g = 0; g < 8; g += M) {
            int cnt = 0;
            for (int j = 0; j < M; ++j)
                cnt += kp[g + j] != 0;
            if (cnt != N)
                bad |= kStatusBadMask;
        }
    } else {
        const u32x4 w = W[u];
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
        for (int d = 0; d < 4; ++d)
            if ((words[d] & 0x7FFFu) > inf_code<DT>() || ((words[d] >> 16) & 0x7FFFu) > inf_code<DT>())
                bad |= kStatusNaN;
    }
    if (bad)
        atomicOr(status, bad);
}

// M is a template parameter so that the group loops unroll and the eight
// words stay in registers (with a run-time M they were indexed dynamically,
// through scratch memory).  With four values a byte (2:4 and 4:8) the kept
// words are gathered by selects and written as one 8-byte store.
template <int DT, int M>
__global__ __launch_bounds__(256) void pack_kernel(const u32x4* __restrict__ W, const uint8_t* __restrict__ keep,
                                                   int64_t nbytes, int N, uint16_t* __restrict__ values,
                                                   uint8_t* __restrict__ masks, const int32_t* __restrict__ rowmap,
                                                   int64_t bpr)
{
    static_assert(M == 4 || M == 8, "groups of 4 or 8 columns");
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nbytes)
        return;
    const int64_t u = source_unit(rowmap, i, bpr);
    const u32x4 wv = W[u];
    uint32_t w[8];
    w[0] = wv.x & 0xFFFF; w[1] = wv.x >> 16; w[2] = wv.y & 0xFFFF; w[3] = wv.y >> 16;
    w[4] = wv.z & 0xFFFF; w[5] = wv.z >> 16; w[6] = wv.w & 0xFFFF; w[7] = wv.w >> 16;
    uint32_t kb = 0;
    if (keep) {
        const uint8_t* kp = keep + 8 * u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            kb |= (uint32_t)(kp[j] != 0) << j;
    } else {
        // Column j is kept when fewer than N group members beat it: larger
        // magnitude, or equal magnitude at a lower column.  For non-NaN words
        // the unsigned order of (bits & 0x7FFF) is the order of |w|.
#pragma unroll
        for (int g = 0; g < 8; g += M) {
#pragma unroll
            for (int j = g; j < g + M; ++j) {
                const uint32_t mj = w[j] & 0x7FFFu;
                int beats = 0;
#pragma unroll
                for (int k = g; k < g + M; ++k) {
                    const uint32_t mk = w[k] & 0x7FFFu;
                    beats += (mk > mj) || (mk == mj && k < j);
                }
                kb |= (uint32_t)(beats < N) << j;
            }
        }
    }
    const int vpb = 8 / M * N;
    masks[i] = (uint8_t)kb;
    if (vpb == 4) {
        // the kept words in column order (the check pass guarantees four; the
        // selects write nothing past the byte's slot whatever the mask holds)
        uint32_t o[4] = {0u, 0u, 0u, 0u};
        int k = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool kept = (kb >> j) & 1u;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                o[t] = (kept && k == t) ? w[j] : o[t];
            k += kept ? 1 : 0;
        }
        // rows are whole bytes, so i * 4 is the fixed-step offset (8-byte aligned)
        *reinterpret_cast<u32x2*>(values + i * 4) = u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
        return;
    }
    uint16_t* out = values + i * vpb;            // rows are whole bytes, so i * vpb is the fixed-step offset
    int k = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (((kb >> j) & 1u) && k < vpb)         // the check pass guarantees k < vpb; the guard keeps writes in bounds
            out[k++] = (uint16_t)w[j];
}

// ---- hybrid sparse + dense rows --------------------------------------------------

// The Spense abstract (fifth page) splits a matrix into a 2:4-sparse and a
// dense region; here the dense region is a set of whole rows, those whose
// pruning loses most.  L_r = sum over the row's pruned columns of w^2 h[c],
// added in column order (groups in column order, pruned columns ascending),
// each term (w*w)*h exact in double and one rounding per added term
// (explicit round-to-nearest operations, no contraction), so the sum is the
// same number the oracle forms.  The pruned columns are those the keep-mask drops,
// or those the top-N magnitude rule (nm_pack's) drops.  Keep-mask groups
// without N kept, or NaN weights under the magnitude rule, set the status
// word (as nm_pack's check does).
constexpr int kLossRows = 32;    // rows per block
constexpr int kLossCols = 64;    // columns per chunk

// Block of 256 threads, 32 rows.  Per 64-column chunk, every thread computes
// the terms of 8 columns (whole groups: M, a template parameter, divides 8) of one row -- thread t
// takes row t / 8, columns 8 (t % 8) .. + 7 -- into LDS with a mask of the
// pruned ones; then thread t < 32 adds its row's pruned terms in column
// order.  Only the adds form a dependent chain; the decoding, the top-N rule
// and the products run in parallel over the chunk (one thread per row and
// column run would leave the chip almost idle: R / 64 waves in all).  32 rows
// a block give R / 32 blocks (448 at R = 14336, so every CU holds work;
// with 64 rows a block, 224 blocks left 32 CUs idle and the rest one block
// each: 0.9 ms for the Llama-3.1-8B gate).
template <int DT, int M>
__global__ __launch_bounds__(256) void hybrid_loss_kernel(const uint16_t* __restrict__ W, const uint8_t* __restrict__ keep,
                                                          const float* __restrict__ h, int64_t h_stride, int R, int K,
                                                          int N, double* __restrict__ loss,
                                                          uint32_t* __restrict__ status)
{
    static_assert(M == 4 || M == 8, "groups of 4 or 8 columns");
    __shared__ double terms[kLossRows][kLossCols + 1];   // +1: the fold's column reads fall in distinct banks
    __shared__ __attribute__((aligned(8))) uint8_t pruned[kLossRows][8];    // bit j of [row][q]: column 8 q + j is pruned
    __shared__ double hs[kLossCols];
    const int t = threadIdx.x;
    const int r0 = blockIdx.x * kLossRows;
    const int lr = t >> 3, q = t & 7, r = r0 + lr;
    const uint16_t* wrow = W + (size_t)(r < R ? r : 0) * K;
    double l = 0.0;
    uint32_t bad = 0;
    // The next chunk's words and h value are loaded while the current one is
    // processed (each chunk otherwise waits for its loads between barriers).
    uint32_t wn[8];
    float hn = 1.f;
    auto fetch = [&](int c0) {
        const int cw = min(kLossCols, K - c0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            wn[j] = (r < R && 8 * q + j < cw) ? wrow[c0 + 8 * q + j] : 0u;
        if (h && t < cw)
            hn = h[(int64_t)(c0 + t) * h_stride];
    };
    fetch(0);
    for (int c0 = 0; c0 < K; c0 += kLossCols) {
        const int cw = min(kLossCols, K - c0);           // a multiple of 8 (K % 8 == 0)
        uint32_t wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            wv[j] = wn[j];
        const float hc = hn;
        if (c0 + kLossCols < K)
            fetch(c0 + kLossCols);
        __syncthreads();                                 // the previous chunk is folded
        if (t < cw)
            hs[t] = h ? nm_decode::f32_to_f64(hc) : 1.0;
        __syncthreads();
        uint32_t pm = 0;
        if (r < R && 8 * q < cw) {
            const uint8_t* kp = keep ? keep + (size_t)r * K + c0 + 8 * q : nullptr;
#pragma unroll
            for (int g = 0; g < 8; g += M) {
                uint32_t kept = 0;
                if (kp) {
                    int cnt = 0;
#pragma unroll
                    for (int j = 0; j < M; ++j) {
                        const uint32_t k = kp[g + j] != 0;
                        kept |= k << j;
                        cnt += (int)k;
                    }
                    if (cnt != N)
                        bad |= kStatusBadMask;
                } else {
#pragma unroll
                    for (int j = 0; j < M; ++j) {
                        const uint32_t mj = wv[g + j] & 0x7FFFu;
                        if (mj > (DT == NM_FP16 ? 0x7C00u : 0x7F80u))
                            bad |= kStatusNaN;
                        int beats = 0;
#pragma unroll
                        for (int k = 0; k < M; ++k) {
                            const uint32_t mk = wv[g + k] & 0x7FFFu;
                            beats += (mk > mj) || (mk == mj && k < j);
                        }
                        kept |= (uint32_t)(beats < N) << j;
                    }
                }
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    if ((kept >> j) & 1u)
                        continue;
                    const double v = nm_decode::w_to_f64<DT>(wv[g + j]);
                    terms[lr][8 * q + g + j] = __dmul_rn(__dmul_rn(v, v), hs[8 * q + g + j]);
                    pm |= 1u << (g + j);
                }
            }
        }
        pruned[lr][q] = (uint8_t)pm;
        __syncthreads();
        if (t < kLossRows && r0 + t < R) {
            const uint64_t pmask = *reinterpret_cast<const uint64_t*>(&pruned[t][0]);   // bit c: column c pruned
            for (int cb = 0; cb < cw; cb += 16) {    // 16 terms read together, then added in order
                double tv[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    tv[j] = terms[t][cb + j];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if ((pmask >> (cb + j)) & 1u)
                        l = __dadd_rn(l, tv[j]);
            }
        }
    }
    if (t < kLossRows && r0 + t < R)
        loss[r0 + t] = l;
    if (bad)
        atomicOr(status, bad);
}

// The ranking order of row losses: every number above NaN (-inf included),
// numbers by value, all NaNs equal.
__device__ __forceinline__ bool loss_above(double a, double b)
{
    return a == a && (b != b || a > b);
}

__device__ __forceinline__ bool loss_equal(double a, double b)
{
    return (a != a) ? (b != b) : (a == b);
}

// flags[r] = 1 for the n_dense rows of largest loss (a NaN loss ranks below
// every number, -inf included; the lower row first among equals): row r's
// rank counts the rows ahead of it, against 256-row tiles of the losses
// staged in LDS.  A block takes 64 rows, four threads per row, each counting
// a quarter of every tile; the four counts add up exactly in any order.
__global__ __launch_bounds__(256) void hybrid_select_kernel(const double* __restrict__ loss, int R, int n_dense,
                                                            uint8_t* __restrict__ flags)
{
    __shared__ double tile[256];
    __shared__ int part[256];
    const int t = threadIdx.x, q = t & 3;
    const int r = blockIdx.x * 64 + (t >> 2);
    const double lr = r < R ? loss[r] : 0.0;
    int above = 0;
    for (int s0 = 0; s0 < R; s0 += 256) {
        __syncthreads();
        if (s0 + t < R)
            tile[t] = loss[s0 + t];
        __syncthreads();
        const int ns = min(256, R - s0);
        for (int k = q; k < ns; k += 4) {
            const double ls = tile[k];
            above += loss_above(ls, lr) || (loss_equal(ls, lr) && s0 + k < r);
        }
    }
    part[t] = above;
    __syncthreads();
    if (q == 0 && r < R)
        flags[r] = part[t] + part[t + 1] + part[t + 2] + part[t + 3] < n_dense ? 1 : 0;
}

// One block: the rows flagged dense, in order, to rows_dense (at most n_dense
// of them are written), the others to rows_sparse (at most R - n_dense); a
// flag count other than n_dense sets the status word.
__global__ __launch_bounds__(1024) void hybrid_partition_kernel(const uint8_t* __restrict__ flags, int R, int n_dense,
                                                                int32_t* __restrict__ rows_sparse,
                                                                int32_t* __restrict__ rows_dense,
                                                                uint32_t* __restrict__ status)
{
    __shared__ int wave_count[1024 / kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, nw = blockDim.x / kWave;
    int dense_before = 0;                        // flagged rows before this pass (block-uniform)
    for (int r0 = 0; r0 < R; r0 += blockDim.x) {
        const int r = r0 + tid;
        const bool f = r < R && flags[r] != 0;
        const uint64_t ball = __ballot(f);
        const int lane_before = __popcll(ball & ((1ull << lane) - 1));
        if (lane == 0)
            wave_count[wave] = __popcll(ball);
        __syncthreads();
        int wave_before = 0, total = 0;
        for (int k = 0; k < nw; ++k) {
            wave_before += k < wave ? wave_count[k] : 0;
            total += wave_count[k];
        }
        if (r < R) {
            const int d = dense_before + wave_before + lane_before;   // flagged rows before r
            if (f) {
                if (d < n_dense)
                    rows_dense[d] = r;
            } else if (r - d < R - n_dense) {
                rows_sparse[r - d] = r;
            }
        }
        dense_before += total;
        __syncthreads();                         // wave_count is rewritten next pass
    }
    if (tid == 0 && dense_before != n_dense)
        atomicOr(status, kStatusBadMask);
}

// W_dense[j] = W[rows_dense[j]], 16-byte units.
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4* __restrict__ W, const int32_t* __restrict__ rows,
                                                          int64_t nunits, int64_t upr, u32x4* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nunits)
        out[i] = W[(int64_t)rows[i / upr] * upr + i % upr];
}

// ---- host: launch helpers ---------------------------------------------------------

// Lets `kernel` take up to the CU's LDS as dynamic shared memory, once per
// kernel and device (the attribute is set for the current device);
// `raised` is the kernel's own array of per-device flags.
int allow_full_lds(const void* kernel, bool* raised)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return NM_ERR_HIP;
    if (!raised[dev]) {
        if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) != hipSuccess)
            return NM_ERR_HIP;
        raised[dev] = true;
    }
    return NM_OK;
}


int hip_status(hipError_t e) { return e == hipSuccess ? NM_OK : NM_ERR_HIP; }


template <int F, int DT, int NT>
int launch_mfma_nt(const Parts& parts, const void* x, int R, int K, int B, hipStream_t s)
{
    const Plan P = plan_mfma_stage<F>(R, K, NT, B);
    if (P.lds > 64 * 1024) {
        static bool raised[64] = {};             // per device, once per instantiation
        if (allow_full_lds((const void*)mfma_stage_kernel<F, DT, NT>, raised) != NM_OK)
            return NM_ERR_HIP;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL((mfma_stage_kernel<F, DT, NT>), dim3(P.grid), dim3(P.threads), P.lds, s, parts,
                       static_cast<const u32x4*>(x), R, K, B, P.S, P.rpb);
    return hip_status(hipGetLastError());
}


template <int F, int DT, int TW, int NT, bool SHX>
int launch_mfma_ring_k(const Plan& P, const Parts& parts, const void* x, int R, int K, int B, hipStream_t s)
{
    if (P.lds > 64 * 1024) {
        static bool raised[64] = {};             // per device, once per instantiation
        if (allow_full_lds((const void*)mfma_ring_kernel<F, DT, TW, NT, SHX>, raised) != NM_OK)
            return NM_ERR_HIP;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL((mfma_ring_kernel<F, DT, TW, NT, SHX>), dim3(P.grid), dim3(P.threads), P.lds, s, parts,
                       static_cast<const u32x4*>(x), R, K, B, P.S, P.rpb, SplitK{},
                       TileMap{(R + 16 * TW - 1) / (16 * TW), P.map_cus, P.map_k});
    return hip_status(hipGetLastError());
}

// K-split ring launch (kind 8) with its workspace: partial sums first, then
// the groups' counters (zero between launches).
template <int F, int DT, int TW, int NT>
int launch_mfma_split(const Plan& P, const Parts& parts, const void* x, int R, int K, int B, hipStream_t s, void* ws)
{
    if (P.lds > 64 * 1024) {
        static bool raised[64] = {};             // per device, once per instantiation
        if (allow_full_lds((const void*)mfma_ring_kernel<F, DT, TW, NT, true, true>, raised) != NM_OK)
            return NM_ERR_HIP;
    }
    uint8_t* w = static_cast<uint8_t*>(ws);
    const SplitK sk{reinterpret_cast<float*>(w), reinterpret_cast<unsigned*>(w + kSplitPartBytes), P.ks, P.kstages};
    (void)hipGetLastError();
    hipLaunchKernelGGL((mfma_ring_kernel<F, DT, TW, NT, true, true>), dim3(P.grid), dim3(P.threads), P.lds, s, parts,
                       static_cast<const u32x4*>(x), R, K, B, 1, P.rpb, sk, TileMap{});
    return hip_status(hipGetLastError());
}

template <int F, int DT, int TW, int NT>
int launch_mfma_ring_tw(const Plan& P, const Parts& parts, const void* x, int R, int K, int B, hipStream_t s)
{
    return P.kind == 7 ? launch_mfma_ring_k<F, DT, TW, NT, true>(P, parts, x, R, K, B, s)
                       : launch_mfma_ring_k<F, DT, TW, NT, false>(P, parts, x, R, K, B, s);
}

// Up to 16 vectors: one batch tile; 17 to 32: two (and two row tiles).
template <int F, int DT>
int launch_mfma_ring(const Parts& parts, const void* x, int R, int K, int B, hipStream_t s)
{
    const Plan P = plan_mfma_ring<F>(R, K, B);
    if (B > 16)
        return launch_mfma_ring_tw<F, DT, 2, 2>(P, parts, x, R, K, B, s);
    return P.cpl == 2 ? launch_mfma_ring_tw<F, DT, 2, 1>(P, parts, x, R, K, B, s)
                      : launch_mfma_ring_tw<F, DT, 1, 1>(P, parts, x, R, K, B, s);
}

// With a workspace, the K-split plan where it applies; else the ring or the
// staged kernel.
template <int F, int DT>
int launch_mfma(const Parts& parts, const void* x, int R, int K, int B, hipStream_t s, void* ws)
{
    Plan SP;
    if (ws && mfma_use_split<F>(R, K, B, &SP)) {
        if (B > 16)
            return launch_mfma_split<F, DT, 2, 2>(SP, parts, x, R, K, B, s, ws);
        return SP.cpl == 2 ? launch_mfma_split<F, DT, 2, 1>(SP, parts, x, R, K, B, s, ws)
                           : launch_mfma_split<F, DT, 1, 1>(SP, parts, x, R, K, B, s, ws);
    }
    if (mfma_use_ring<F>(R, K, B))
        return launch_mfma_ring<F, DT>(parts, x, R, K, B, s);
    return B > 16 ? launch_mfma_nt<F, DT, 2>(parts, x, R, K, B, s) : launch_mfma_nt<F, DT, 1>(parts, x, R, K, B, s);
}

// ws: the caller's K-split workspace (kSplitWorkspaceBytes, counters zero), or NULL.
template <int F>
int launch_mfma_dt(int dtype, const Parts* parts, const void* x, int R, int K, int B, hipStream_t s,
                   void* ws = nullptr)
{
    return dtype == NM_FP16 ? launch_mfma<F, NM_FP16>(*parts, x, R, K, B, s, ws)
                            : launch_mfma<F, NM_BF16>(*parts, x, R, K, B, s, ws);
}

// Launches the chosen kernel over the concatenated rows of `parts` (R in total).
template <int F, int DT, int NB>
int launch_rows(const Parts& parts, const void* x, int R, int K, hipStream_t s)
{
    const Plan P = plan_for<F>(R, K, NB, parts.glu != 0);
    const u32x4* x4 = static_cast<const u32x4*>(x);
    (void)hipGetLastError();
    if (P.kind == 1) {
        const int xu = rowslice_x_regs(NB, K, P.threads, P.cpl);
#define NM_SLICE_XU(CPL, XU)                                                                                         \
    hipLaunchKernelGGL((rowslice_kernel<F, DT, NB, CPL, XU>), dim3(P.grid), dim3(P.threads), P.lds, s, parts, x4, R, \
                       K, P.ls, P.rpb, P.xf, (int)(xu != 0))
#define NM_SLICE(CPL)                  \
    do {                               \
        if constexpr (NB == 1) {       \
            if (xu == 4)               \
                NM_SLICE_XU(CPL, 4);   \
            else                       \
                NM_SLICE_XU(CPL, 1);   \
        } else {                       \
            NM_SLICE_XU(CPL, 1);       \
        }                              \
    } while (0)
        if constexpr (NB <= 4 && F != kDense) {
            // row pairs (two rows a wave; the plan takes them at 4 or 5 chunks a lane)
            if (P.rpw == 2) {
                if (xu > 1)                      // the plan never pairs rows whose x needs more
                    return NM_ERR_UNSUPPORTED;
                if (P.cpl == 4)
                    hipLaunchKernelGGL((rowslice_kernel<F, DT, NB, 4, 1, 2>), dim3(P.grid), dim3(P.threads), P.lds, s,
                                       parts, x4, R, K, P.ls, P.rpb, P.xf, (int)(xu != 0));
                else
                    hipLaunchKernelGGL((rowslice_kernel<F, DT, NB, 5, 1, 2>), dim3(P.grid), dim3(P.threads), P.lds, s,
                                       parts, x4, R, K, P.ls, P.rpb, P.xf, (int)(xu != 0));
                return hip_status(hipGetLastError());
            }
        }
        if constexpr (NB == 1 && F != kDense) {
            // long rows on one wave (single vector): the next even slot count
            if (P.cpl > 8) {
                if (P.cpl <= 10)
                    NM_SLICE_XU(10, 1);
                else if (P.cpl <= 12)
                    NM_SLICE_XU(12, 1);
                else if (P.cpl <= 14)
                    NM_SLICE_XU(14, 1);
                else
                    NM_SLICE_XU(16, 1);
                return hip_status(hipGetLastError());
            }
        }
        switch (P.cpl) {
        case 1: NM_SLICE(1); break;
        case 2: NM_SLICE(2); break;
        case 3: NM_SLICE(3); break;
        case 4: NM_SLICE(4); break;
        case 5: NM_SLICE(5); break;
        case 6: NM_SLICE(6); break;
        case 7: NM_SLICE(7); break;
        default: NM_SLICE(8); break;
        }
#undef NM_SLICE
#undef NM_SLICE_XU
    } else {
        if (P.lds > 64 * 1024) {
            static bool raised[64] = {};         // per device, once per instantiation
            if (allow_full_lds((const void*)stream_kernel<F, DT, NB, 4>, raised) != NM_OK)
                return NM_ERR_HIP;
        }
        hipLaunchKernelGGL((stream_kernel<F, DT, NB, 4>), dim3(P.grid), dim3(P.threads), P.lds, s, parts, x4, R, K,
                           P.tile_cols);
    }
    return hip_status(hipGetLastError());
}

// A hybrid matrix's sparse rows (PS, RS of them) and dense rows (PD, RD) at NB
// x vectors (1 to 3: where both parts run on the row-slice kernel) in one
// hybrid_rowslice_kernel launch.  It applies when the sparse rows get a
// row-slice plan (taken with at least two rows per block) with an even number
// of rows per block (the dense rows take half as many, over twice the
// slices); *launched is false, and nothing is launched, otherwise.
template <int F, int DT, int NB>
int launch_hybrid_fused(const Parts& PS, const Parts& PD, const void* x, int RS, int RD, int K, hipStream_t s,
                        bool* launched)
{
    *launched = false;
    Plan P;
    if (!plan_hybrid<F>(RS, K, NB, &P))
        return NM_OK;
    const int64_t dense_rpb = P.rpb / 2;
    const int64_t sblocks = P.grid, blocks = sblocks + (RD + dense_rpb - 1) / dense_rpb;
    const u32x4* x4 = static_cast<const u32x4*>(x);
    (void)hipGetLastError();
#define NM_HYB(CPL)                                                                                             \
    hipLaunchKernelGGL((hybrid_rowslice_kernel<F, DT, NB, CPL, 1>), dim3((unsigned)blocks), dim3(P.threads), P.lds, s, \
                       PS, PD, x4, RS, RD, K, P.ls, P.rpb, P.xf, (int)(NB * (K / 8) <= P.threads), (int)sblocks)
    switch (P.cpl) {
    case 1: NM_HYB(1); break;
    case 2: NM_HYB(2); break;
    case 3: NM_HYB(3); break;
    case 4: NM_HYB(4); break;
    case 5: NM_HYB(5); break;
    case 6: NM_HYB(6); break;
    case 7: NM_HYB(7); break;
    default: NM_HYB(8); break;
    }
#undef NM_HYB
    *launched = true;
    return hip_status(hipGetLastError());
}

template <int F, int DT>
int launch_hybrid_fused_nb(int B, const Parts& PS, const Parts& PD, const void* x, int RS, int RD, int K,
                           hipStream_t s, bool* launched)
{
    switch (B) {
    case 1: return launch_hybrid_fused<F, DT, 1>(PS, PD, x, RS, RD, K, s, launched);
    case 2: return launch_hybrid_fused<F, DT, 2>(PS, PD, x, RS, RD, K, s, launched);
    case 3: return launch_hybrid_fused<F, DT, 3>(PS, PD, x, RS, RD, K, s, launched);
    default: *launched = false; return NM_OK;
    }
}

template <int F>
int launch_hybrid_fused_dt(int dtype, int B, const Parts& PS, const Parts& PD, const void* x, int RS, int RD, int K,
                           hipStream_t s, bool* launched)
{
    return dtype == NM_FP16 ? launch_hybrid_fused_nb<F, NM_FP16>(B, PS, PD, x, RS, RD, K, s, launched)
                            : launch_hybrid_fused_nb<F, NM_BF16>(B, PS, PD, x, RS, RD, K, s, launched);
}

int launch_zero(void* y, int64_t n, hipStream_t s)
{
    if (n == 0)
        return NM_OK;
    (void)hipGetLastError();
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint16_t*)y, n);
    return hip_status(hipGetLastError());
}

// ---- host: dtype x batch dispatch ------------------------------------------------

template <template <int, int> class Fn, typename... A>
int dispatch(int dtype, int B, A... a)
{
#define NM_CASES(DT)                            \
    switch (B) {                                \
    case 1: return Fn<DT, 1>::run(a...);        \
    case 2: return Fn<DT, 2>::run(a...);        \
    case 3: return Fn<DT, 3>::run(a...);        \
    case 4: return Fn<DT, 4>::run(a...);        \
    case 5: return Fn<DT, 5>::run(a...);        \
    case 6: return Fn<DT, 6>::run(a...);        \
    case 7: return Fn<DT, 7>::run(a...);        \
    case 8: return Fn<DT, 8>::run(a...);        \
    }
    if (dtype == NM_FP16) {
        NM_CASES(NM_FP16)
    } else {
        NM_CASES(NM_BF16)
    }
#undef NM_CASES
    return NM_ERR_BAD_SHAPE;
}

template <int DT, int NB>
struct Sparse24 {
    static int run(const Parts* p, const void* x, int R, int K, hipStream_t s)
    {
        return launch_rows<kNM24, DT, NB>(*p, x, R, K, s);
    }
};

template <int DT, int NB>
struct Sparse48 {
    static int run(const Parts* p, const void* x, int R, int K, hipStream_t s)
    {
        return launch_rows<kNM48, DT, NB>(*p, x, R, K, s);
    }
};

template <int DT, int NB>
struct SparseGeneric {
    static int run(const void* v, const uint8_t* m, const void* v2, const uint8_t* m2, const void* x, void* y, int R,
                   int K, int N, int M, const int32_t* ymap, int ystride, hipStream_t s)
    {
        (void)hipGetLastError();
        const unsigned grid = (unsigned)((R + 3) / 4);
        hipLaunchKernelGGL((generic_spmv_kernel<DT, NB>), dim3(grid), dim3(256), 0, s, (const uint16_t*)v, m,
                           (const uint16_t*)v2, m2, (const uint16_t*)x, (uint16_t*)y, R, K, N, M, ymap, ystride);
        return hip_status(hipGetLastError());
    }
};

template <int DT, int NB>
struct Dense {
    static int run(const Parts* p, const void* x, int R, int K, hipStream_t s)
    {
        return launch_rows<kDense, DT, NB>(*p, x, R, K, s);
    }
};

// nm_pack's error word lives in device memory, one per GPU; its address comes
// from hipGetSymbolAddress (never the symbol's host-side name).
__device__ uint32_t g_pack_status;
std::mutex g_pack_mutex;
uint32_t* g_status_ptr[64] = {};

int status_word(uint32_t** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return NM_ERR_HIP;
    if (!g_status_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_pack_status)) != hipSuccess || !p)
            return NM_ERR_HIP;
        g_status_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_status_ptr[dev];
    return NM_OK;
}

// The generic kernel takes at most 8 vectors per launch: larger batches go
// through it 8 rows of x (and y) at a time.  ymap / ystride as in Parts.
int generic_batches(int dtype, int B, const void* v, const uint8_t* m, const void* v2, const uint8_t* m2, const void* x,
                    void* y, int64_t R, int64_t K, int N, int M, hipStream_t s, const int32_t* ymap = nullptr,
                    int ystride = 0)
{
    const int64_t ys = ymap ? ystride : R;
    for (int b0 = 0; b0 < B; b0 += kVectorMaxBatch) {
        const int nb = std::min(kVectorMaxBatch, B - b0);
        const void* xb = static_cast<const uint16_t*>(x) + (size_t)b0 * (size_t)K;
        void* yb = static_cast<uint16_t*>(y) + (size_t)b0 * (size_t)ys;
        const int st = dispatch<SparseGeneric>(dtype, nb, v, m, v2, m2, xb, yb, (int)R, (int)K, N, M, ymap, ystride, s);
        if (st != NM_OK)
            return st;
    }
    return NM_OK;
}

// Pack R_out rows (output row o from source row rowmap[o], or o itself):
// check every group first (status word, synchronous), then pack; returns
// when the outputs are complete.  Arguments are already validated.
int pack_rows(const void* W, const uint8_t* keep, const int32_t* rowmap, int64_t R, int64_t K, int N, int M, int dtype,
              void* values, uint8_t* masks, hipStream_t s)
{
    int st = NM_OK;
    const int64_t nbytes = R * (K / 8);
    if (nbytes == 0)
        return NM_OK;
    std::lock_guard<std::mutex> lock(g_pack_mutex);
    uint32_t* status = nullptr;
    if ((st = status_word(&status)) != NM_OK)
        return st;
    const unsigned grid = (unsigned)((nbytes + 255) / 256);
    (void)hipGetLastError();
    if (hipMemsetAsync(status, 0, sizeof(uint32_t), s) != hipSuccess)
        return NM_ERR_HIP;
    if (dtype == NM_FP16)
        hipLaunchKernelGGL(pack_check_kernel<NM_FP16>, dim3(grid), dim3(256), 0, s, (const u32x4*)W, keep, nbytes, N, M,
                           status, rowmap, K / 8);
    else
        hipLaunchKernelGGL(pack_check_kernel<NM_BF16>, dim3(grid), dim3(256), 0, s, (const u32x4*)W, keep, nbytes, N, M,
                           status, rowmap, K / 8);
    if (hipGetLastError() != hipSuccess)
        return NM_ERR_HIP;
    uint32_t host_status = 0;
    if (hipMemcpyAsync(&host_status, status, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return NM_ERR_HIP;
    if (host_status & kStatusBadMask)
        return NM_ERR_BAD_MASK;
    if (host_status & kStatusNaN)
        return NM_ERR_NONFINITE;
#define NM_PACK(DT, MM)                                                                                          \
    hipLaunchKernelGGL((pack_kernel<DT, MM>), dim3(grid), dim3(256), 0, s, (const u32x4*)W, keep, nbytes, N,       \
                       (uint16_t*)values, masks, rowmap, K / 8)
    if (dtype == NM_FP16) {
        if (M == 4)
            NM_PACK(NM_FP16, 4);
        else
            NM_PACK(NM_FP16, 8);
    } else {
        if (M == 4)
            NM_PACK(NM_BF16, 4);
        else
            NM_PACK(NM_BF16, 8);
    }
#undef NM_PACK
    if (hipGetLastError() != hipSuccess)
        return NM_ERR_HIP;
    return hip_status(hipStreamSynchronize(s));
}

// Enqueues `launch(status)` (kernels that may set status bits), waits, and
// translates the bits: a bad keep-mask or row count -> NM_ERR_BAD_MASK, a NaN
// under the magnitude rule -> NM_ERR_NONFINITE.
template <typename Fn>
int with_status(hipStream_t s, Fn launch)
{
    std::lock_guard<std::mutex> lock(g_pack_mutex);
    uint32_t* status = nullptr;
    int st = status_word(&status);
    if (st != NM_OK)
        return st;
    (void)hipGetLastError();
    if (hipMemsetAsync(status, 0, sizeof(uint32_t), s) != hipSuccess)
        return NM_ERR_HIP;
    launch(status);
    if (hipGetLastError() != hipSuccess)
        return NM_ERR_HIP;
    uint32_t host_status = 0;
    if (hipMemcpyAsync(&host_status, status, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return NM_ERR_HIP;
    if (host_status & kStatusBadMask)
        return NM_ERR_BAD_MASK;
    if (host_status & kStatusNaN)
        return NM_ERR_NONFINITE;
    return NM_OK;
}

// One part of a hybrid matrix (sparse rows or dense rows), scattered into y.
Parts mapped_part(const void* w, const uint8_t* m, const int32_t* rows, int64_t Rp, int64_t R, void* y)
{
    Parts P = {};
    P.w[0] = static_cast<const u32x4*>(w);
    P.m[0] = reinterpret_cast<const uint16_t*>(m);
    P.y[0] = static_cast<uint16_t*>(y);
    P.ymap[0] = rows;
    P.ystride[0] = (int)R;
    P.count = 1;
    for (int i = 1; i <= kMaxParts; ++i)
        P.begin[i] = (int)Rp;
    return P;
}

}  // namespace

// Compute units of the current device, read once per device (256 if the
// runtime cannot say).
int nmh::cu_count()
{
    static int counts[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!counts[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        counts[dev] = n;
    }
    return counts[dev];
}

// ---- the allocation-free workspace ---------------------------------------------------

namespace {

// The K-split workspace of nm_spmv_multi_noalloc: one array per GPU, in the
// library's code object (zero when loaded), shared by every such call on that
// GPU.  Host code never names it as an address: its device address is taken
// once per device with hipGetSymbolAddress.
__device__ __align__(256) uint8_t scratch[kSplitWorkspaceBytes];

std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[64] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

}  // namespace

int nmk::static_workspace(void** out, void* stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return NM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return NM_ERR_HIP;
        // The counters start at zero (and every completed launch leaves them
        // there); clear them once more on this device's first call, by a kernel
        // on the caller's stream (captured with it, if the call is captured).
        (void)hipGetLastError();
        hipLaunchKernelGGL(zero_words_kernel, dim3((kSplitMaxGroups + 255) / 256), dim3(256), 0,
                           static_cast<hipStream_t>(stream),
                           reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p) + kSplitPartBytes), kSplitMaxGroups);
        if (hipGetLastError() != hipSuccess)
            return NM_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return NM_OK;
}

// ---- the kernel side of the entry points (arguments checked by nmapi.cpp) --------

int nmk::zero(void* y, int64_t n, void* stream) { return launch_zero(y, n, static_cast<hipStream_t>(stream)); }

int nmk::spmv_multi(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t total,
                    int64_t K, int N, int M, int dtype, const void* x, int B, void* const* y, void* workspace,
                    void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K % 16 == 0 && ((N == 2 && M == 4) || (N == 4 && M == 8))) {
        Parts P = {};
        P.begin[0] = 0;
        for (int i = 0; i < count; ++i) {
            if (R[i] == 0)
                continue;
            P.w[P.count] = static_cast<const u32x4*>(values[i]);
            P.m[P.count] = reinterpret_cast<const uint16_t*>(masks[i]);
            P.y[P.count] = static_cast<uint16_t*>(y[i]);
            P.begin[P.count + 1] = P.begin[P.count] + (int)R[i];
            ++P.count;
        }
        for (int i = P.count + 1; i <= kMaxParts; ++i)
            P.begin[i] = P.begin[P.count];
        if (M == 4 ? use_mfma<kNM24>(total, K, B, false) : use_mfma<kNM48>(total, K, B, false))
            return M == 4 ? launch_mfma_dt<kNM24>(dtype, &P, x, (int)total, (int)K, B, s, workspace)
                          : launch_mfma_dt<kNM48>(dtype, &P, x, (int)total, (int)K, B, s, workspace);
        return M == 4 ? dispatch<Sparse24>(dtype, B, (const Parts*)&P, x, (int)total, (int)K, s)
                      : dispatch<Sparse48>(dtype, B, (const Parts*)&P, x, (int)total, (int)K, s);
    }
    for (int i = 0; i < count; ++i) {
        if (R[i] == 0)
            continue;
        const int st = generic_batches(dtype, B, values[i], masks[i], nullptr, nullptr, x, y[i], R[i], K, N, M, s);
        if (st != NM_OK)
            return st;
    }
    return NM_OK;
}

int nmk::gemv_dense_multi(int count, const void* const* W, const int64_t* R, int64_t total, int64_t K, int dtype,
                          const void* x, int B, void* const* y, void* workspace, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    Parts P = {};
    for (int i = 0; i < count; ++i) {
        if (R[i] == 0)
            continue;
        P.w[P.count] = static_cast<const u32x4*>(W[i]);
        P.m[P.count] = nullptr;
        P.y[P.count] = static_cast<uint16_t*>(y[i]);
        P.begin[P.count + 1] = P.begin[P.count] + (int)R[i];
        ++P.count;
    }
    for (int i = P.count + 1; i <= kMaxParts; ++i)
        P.begin[i] = P.begin[P.count];
    if (use_mfma<kDense>(total, K, B, false))
        return launch_mfma_dt<kDense>(dtype, &P, x, (int)total, (int)K, B, s, workspace);
    return dispatch<Dense>(dtype, B, (const Parts*)&P, x, (int)total, (int)K, s);
}

int nmk::spmv_swiglu(const void* values_gate, const uint8_t* masks_gate, const void* values_up,
                     const uint8_t* masks_up, int64_t R, int64_t K, int N, int M, int dtype, const void* x, int B,
                     void* h, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K % 16 == 0 && ((N == 2 && M == 4) || (N == 4 && M == 8))) {
        Parts P = {};
        P.w[0] = static_cast<const u32x4*>(values_gate);
        P.m[0] = reinterpret_cast<const uint16_t*>(masks_gate);
        P.w[1] = static_cast<const u32x4*>(values_up);
        P.m[1] = reinterpret_cast<const uint16_t*>(masks_up);
        P.y[0] = static_cast<uint16_t*>(h);
        P.count = 2;
        P.glu = 1;
        P.begin[1] = (int)R;
        for (int i = 2; i <= kMaxParts; ++i)
            P.begin[i] = (int)(2 * R);
        if (M == 4 ? use_mfma<kNM24>(2 * R, K, B, true) : use_mfma<kNM48>(2 * R, K, B, true))
            return M == 4 ? launch_mfma_dt<kNM24>(dtype, &P, x, (int)(2 * R), (int)K, B, s)
                          : launch_mfma_dt<kNM48>(dtype, &P, x, (int)(2 * R), (int)K, B, s);
        return M == 4 ? dispatch<Sparse24>(dtype, B, (const Parts*)&P, x, (int)(2 * R), (int)K, s)
                      : dispatch<Sparse48>(dtype, B, (const Parts*)&P, x, (int)(2 * R), (int)K, s);
    }
    return generic_batches(dtype, B, values_gate, masks_gate, values_up, masks_up, x, h, R, K, N, M, s);
}

int nmk::gemv_dense_swiglu(const void* W_gate, const void* W_up, int64_t R, int64_t K, int dtype, const void* x,
                           int B, void* h, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    Parts P = {};
    P.w[0] = static_cast<const u32x4*>(W_gate);
    P.w[1] = static_cast<const u32x4*>(W_up);
    P.y[0] = static_cast<uint16_t*>(h);
    P.count = 2;
    P.glu = 1;
    P.begin[1] = (int)R;
    for (int i = 2; i <= kMaxParts; ++i)
        P.begin[i] = (int)(2 * R);
    if (use_mfma<kDense>(2 * R, K, B, true))
        return launch_mfma_dt<kDense>(dtype, &P, x, (int)(2 * R), (int)K, B, s);
    return dispatch<Dense>(dtype, B, (const Parts*)&P, x, (int)(2 * R), (int)K, s);
}

int nmk::pack(const void* W, const uint8_t* keep, int64_t R, int64_t K, int N, int M, int dtype, void* values,
              uint8_t* masks, void* stream)
{
    return pack_rows(W, keep, nullptr, R, K, N, M, dtype, values, masks, static_cast<hipStream_t>(stream));
}

int nmk::hybrid_row_loss(const void* W, const uint8_t* keep, const float* h, int64_t h_stride, int64_t R, int64_t K,
                         int N, int M, int dtype, double* loss, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned grid = (unsigned)((R + kLossRows - 1) / kLossRows);
    return with_status(s, [&](uint32_t* status) {
#define NM_LOSS(DT, MM)                                                                                        \
    hipLaunchKernelGGL((hybrid_loss_kernel<DT, MM>), dim3(grid), dim3(256), 0, s, (const uint16_t*)W, keep, h,  \
                       h_stride, (int)R, (int)K, N, loss, status)
        if (dtype == NM_FP16) {
            if (M == 4)
                NM_LOSS(NM_FP16, 4);
            else
                NM_LOSS(NM_FP16, 8);
        } else {
            if (M == 4)
                NM_LOSS(NM_BF16, 4);
            else
                NM_LOSS(NM_BF16, 8);
        }
#undef NM_LOSS
    });
}

int nmk::hybrid_select_rows(const double* loss, int64_t R, int64_t n_dense, uint8_t* flags, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipLaunchKernelGGL(hybrid_select_kernel, dim3((unsigned)((R + 63) / 64)), dim3(256), 0, s, loss, (int)R,
                       (int)n_dense, flags);
    return hip_status(hipGetLastError());
}

int nmk::hybrid_pack(const void* W, const uint8_t* keep, const uint8_t* flags, int64_t n_dense, int64_t R, int64_t K,
                     int N, int M, int dtype, void* values, uint8_t* masks, void* W_dense, int32_t* rows_sparse,
                     int32_t* rows_dense, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t Rs = R - n_dense;
    int st = with_status(s, [&](uint32_t* status) {
        hipLaunchKernelGGL(hybrid_partition_kernel, dim3(1), dim3(1024), 0, s, flags, (int)R, (int)n_dense, rows_sparse,
                           rows_dense, status);
    });
    if (st != NM_OK)
        return st;
    if (K == 0)
        return NM_OK;
    if ((st = pack_rows(W, keep, rows_sparse, Rs, K, N, M, dtype, values, masks, s)) != NM_OK)
        return st;
    const int64_t upr = K / 8, nunits = n_dense * upr;
    if (nunits > 0) {
        (void)hipGetLastError();
        hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((nunits + 255) / 256)), dim3(256), 0, s,
                           static_cast<const u32x4*>(W), rows_dense, nunits, upr, static_cast<u32x4*>(W_dense));
        if (hipGetLastError() != hipSuccess)
            return NM_ERR_HIP;
    }
    return hip_status(hipStreamSynchronize(s));
}

int nmk::spmv_hybrid(const void* values, const uint8_t* masks, const int32_t* rows_sparse, const void* W_dense,
                     const int32_t* rows_dense, int64_t n_dense, int64_t R, int64_t K, int N, int M, int dtype,
                     const void* x, int B, void* y, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t Rs = R - n_dense;
    int st = NM_OK;
    const bool tuned = K % 16 == 0 && ((N == 2 && M == 4) || (N == 4 && M == 8));
    if (B <= 3 && Rs > 0 && n_dense > 0 && tuned) {
        std::call_once(g_env_once, read_env);
        if (g_env.hybrid_split != 1) {
            const Parts PS = mapped_part(values, masks, rows_sparse, Rs, R, y);
            const Parts PD = mapped_part(W_dense, nullptr, rows_dense, n_dense, R, y);
            bool launched = false;
            st = M == 4 ? launch_hybrid_fused_dt<kNM24>(dtype, B, PS, PD, x, (int)Rs, (int)n_dense, (int)K, s, &launched)
                        : launch_hybrid_fused_dt<kNM48>(dtype, B, PS, PD, x, (int)Rs, (int)n_dense, (int)K, s,
                                                        &launched);
            if (launched || st != NM_OK)
                return st;
        }
    }
    if (Rs > 0) {
        const Parts P = mapped_part(values, masks, rows_sparse, Rs, R, y);
        if (tuned) {
            if (M == 4 ? use_mfma<kNM24>(Rs, K, B, false) : use_mfma<kNM48>(Rs, K, B, false))
                st = M == 4 ? launch_mfma_dt<kNM24>(dtype, &P, x, (int)Rs, (int)K, B, s)
                            : launch_mfma_dt<kNM48>(dtype, &P, x, (int)Rs, (int)K, B, s);
            else
                st = M == 4 ? dispatch<Sparse24>(dtype, B, &P, x, (int)Rs, (int)K, s)
                            : dispatch<Sparse48>(dtype, B, &P, x, (int)Rs, (int)K, s);
        } else {
            st = generic_batches(dtype, B, values, masks, nullptr, nullptr, x, y, Rs, K, N, M, s, rows_sparse, (int)R);
        }
        if (st != NM_OK)
            return st;
    }
    if (n_dense > 0) {
        const Parts P = mapped_part(W_dense, nullptr, rows_dense, n_dense, R, y);
        if (use_mfma<kDense>(n_dense, K, B, false))
            return launch_mfma_dt<kDense>(dtype, &P, x, (int)n_dense, (int)K, B, s);
        return dispatch<Dense>(dtype, B, &P, x, (int)n_dense, (int)K, s);
    }
    return NM_OK;
}

