// nmspmv.hip -- libnmspmv: N:M sparse matrix-vector products on gfx950.
//
// The decode-time hot path named by "SparseDecoding: Decoding-Aware Pruning
// for Accurate and Efficient LLM Inference" (humanity-list story page,
// "Abstract"): an N:M sparse matrix-vector kernel with bitmask indexing and
// fixed-step traversal, used because decoding is memory-bound and the weight
// bytes read per token set the time.  The pages' kernel was written for A100;
// this one is designed for CDNA4 (wave64, 160 KB LDS per CU, HBM3E) and shares
// nothing with the CPU checker.
//
// Format (see include/nmspmv.h): values [R][K*N/M] 16-bit, group g of a row at
// value g*N; masks [R][K/8] one bit per dense column, LSB first.
//
// Kernels
//   rowdot_kernel<SPARSE=true>   N/M = 1/2 (2:4, 4:8), K % 16 == 0.  Each lane
//       streams 16-byte chunks of a row's values (8 values = 16 dense columns)
//       plus the 16 mask bits of those columns, expands the 8 values into the
//       16 dense columns with 8 byte-permutes whose selectors come from a
//       256-entry LDS table indexed by mask byte, and multiplies against x
//       staged in LDS with packed dot2 (fp32 accumulate).
//   rowdot_kernel<SPARSE=false>  dense GEMV baseline, same skeleton, 16-byte
//       chunks of W (8 columns).
//   generic_spmv_kernel          any N:M (M = 4 or 8) and K % 8 == 0: one mask
//       byte per lane step, values read word by word.  Correct, not tuned.
//   pack_check_kernel / pack_kernel   nm_pack's validation and packing passes.
// Rows are owned by wavefronts; each row's partial sums are reduced across the
// 64 lanes with DPP row permutes and four lane reads (fixed order, so results
// are deterministic run to run).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "nmspmv.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kUnroll = 4;                       // 16-byte chunks in flight per lane per row step
constexpr int kXTileBudget = 56 * 1024;          // bytes of LDS for the staged x tile

// ---- arithmetic helpers --------------------------------------------------

// fp32 += a.lo * b.lo + a.hi * b.hi for two packed 16-bit pairs.  Products of
// two 16-bit floats are exact in fp32.
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
    float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (a + b) + (c + d);
}

// Byte-permute selectors that expand the four 16-bit values of one mask byte
// (8 dense columns) into four dense dwords.  Value k (in column order) sits in
// bytes 2k, 2k+1 of the 8-byte source {hi dword : lo dword}; an unkept column
// gets selector 0x0C, which v_perm_b32 turns into a zero byte.  With more than
// four bits set (a malformed mask) selectors run past 7 and produce junk
// bytes, never an out-of-range access.
__device__ u32x4 expand_selectors(uint32_t mb)
{
    uint32_t s[4];
    uint32_t k = 0;
    for (int d = 0; d < 4; ++d) {
        uint32_t sel = 0;
        for (int h = 0; h < 2; ++h) {
            int j = 2 * d + h;
            uint32_t pair = 0x0C0Cu;
            if ((mb >> j) & 1u) {
                pair = (2 * k) | ((2 * k + 1) << 8);
                ++k;
            }
            sel |= pair << (16 * h);
        }
        s[d] = sel;
    }
    return u32x4{s[0], s[1], s[2], s[3]};
}

// ---- row-dot kernels (sparse N/M = 1/2 and dense) -------------------------

// One block owns rows [blockIdx.x * rows_per_block, +rows_per_block); its
// waves take those rows round-robin.  x is staged into LDS in tiles of
// tile_cols columns (one tile when B*K*2 bytes fit); with several tiles the
// per-row partial sums wait in LDS between tiles.
template <bool SPARSE, int DT, int NB>
__global__ __launch_bounds__(kBlock) void rowdot_kernel(const u32x4* __restrict__ w4, const uint16_t* __restrict__ m2,
                                                        const u32x4* __restrict__ x4, uint16_t* __restrict__ y, int R,
                                                        int K, int rows_per_block, int tile_cols)
{
    extern __shared__ u32x4 smem[];
    constexpr int COLS = SPARSE ? 16 : 8;        // dense columns per 16-byte chunk
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r0 = blockIdx.x * rows_per_block;
    const int r1 = min(R, r0 + rows_per_block);
    const int tq = tile_cols / 8;                // 16-byte x chunks per batch row of the tile
    u32x4* lut = smem;
    u32x4* xs = smem + (SPARSE ? 256 : 0);
    float* part = reinterpret_cast<float*>(xs + NB * tq);
    const bool multi = tile_cols < K;
    const int cpr = K / COLS;

    if constexpr (SPARSE)
        lut[threadIdx.x] = expand_selectors(threadIdx.x);
    if (multi)
        for (int i = threadIdx.x; i < rows_per_block * NB; i += kBlock)
            part[i] = 0.f;

    for (int t0 = 0; t0 < K; t0 += tile_cols) {
        const int tc = min(tile_cols, K - t0);
        __syncthreads();
        const int q = tc / 8;
        for (int i = threadIdx.x; i < NB * q; i += kBlock) {
            int b = i / q, j = i - b * q;
            xs[b * tq + j] = x4[(size_t)b * (K / 8) + t0 / 8 + j];
        }
        __syncthreads();
        const int cb = t0 / COLS, ce = (t0 + tc) / COLS;
        for (int r = r0 + wave; r < r1; r += kWavesPerBlock) {
            float acc[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[b] = 0.f;
            const u32x4* wrow = w4 + (size_t)r * cpr;
            const uint16_t* mrow = m2 + (size_t)r * cpr;
            for (int c0 = cb; c0 < ce; c0 += kWave * kUnroll) {
                u32x4 v[kUnroll];
                uint32_t mk[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int c = c0 + u * kWave + lane;
                    v[u] = u32x4{0, 0, 0, 0};
                    mk[u] = 0;
                    if (c < ce) {
                        v[u] = __builtin_nontemporal_load(wrow + c);
                        if constexpr (SPARSE)
                            mk[u] = __builtin_nontemporal_load(mrow + c);
                    }
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int c = c0 + u * kWave + lane;
                    if (c >= ce)
                        continue;
                    const int xi = (c * COLS - t0) / 8;      // first 16-byte x chunk of this column range
                    if constexpr (SPARSE) {
                        const u32x4 s0 = lut[mk[u] & 0xFF];
                        const u32x4 s1 = lut[mk[u] >> 8];
                        uint32_t w[8];
                        w[0] = __builtin_amdgcn_perm(v[u].y, v[u].x, s0.x);
                        w[1] = __builtin_amdgcn_perm(v[u].y, v[u].x, s0.y);
                        w[2] = __builtin_amdgcn_perm(v[u].y, v[u].x, s0.z);
                        w[3] = __builtin_amdgcn_perm(v[u].y, v[u].x, s0.w);
                        w[4] = __builtin_amdgcn_perm(v[u].w, v[u].z, s1.x);
                        w[5] = __builtin_amdgcn_perm(v[u].w, v[u].z, s1.y);
                        w[6] = __builtin_amdgcn_perm(v[u].w, v[u].z, s1.z);
                        w[7] = __builtin_amdgcn_perm(v[u].w, v[u].z, s1.w);
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            const u32x4 xa = xs[b * tq + xi];
                            const u32x4 xb = xs[b * tq + xi + 1];
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
                    } else {
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            const u32x4 xa = xs[b * tq + xi];
                            float a = acc[b];
                            a = dot2<DT>(v[u].x, xa.x, a);
                            a = dot2<DT>(v[u].y, xa.y, a);
                            a = dot2<DT>(v[u].z, xa.z, a);
                            a = dot2<DT>(v[u].w, xa.w, a);
                            acc[b] = a;
                        }
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float s = wave_sum(acc[b]);
                if (lane == 0) {
                    if (multi)
                        part[(r - r0) * NB + b] += s;
                    else
                        y[(size_t)b * R + r] = from_f32<DT>(s);
                }
            }
        }
    }
    if (multi) {
        __syncthreads();
        for (int i = threadIdx.x; i < (r1 - r0) * NB; i += kBlock) {
            const int row = i / NB, b = i - row * NB;
            y[(size_t)b * R + r0 + row] = from_f32<DT>(part[i]);
        }
    }
}

// ---- generic N:M (any N < M, M in {4, 8}, K % 8 == 0) --------------------

template <int DT, int NB>
__global__ __launch_bounds__(kBlock) void generic_spmv_kernel(const uint16_t* __restrict__ values,
                                                              const uint8_t* __restrict__ masks,
                                                              const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                              int R, int K, int N, int M)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (row >= R)                                // whole wave leaves together
        return;
    const int vpb = 8 / M * N;                   // values per mask byte (fixed step)
    const size_t vrow = (size_t)(K / M) * N;
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        acc[b] = 0.f;
    for (int q = lane; q < K / 8; q += kWave) {
        const uint32_t mb = masks[(size_t)row * (K / 8) + q];
        const uint16_t* vp = values + (size_t)row * vrow + (size_t)q * vpb;
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
    for (int b = 0; b < NB; ++b) {
        const float s = wave_sum(acc[b]);
        if (lane == 0)
            y[(size_t)b * R + row] = from_f32<DT>(s);
    }
}

__global__ void fill_zero_kernel(uint16_t* __restrict__ y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        y[i] = 0;
}

// ---- pack -------------------------------------------------------------------

constexpr uint32_t kStatusBadMask = 1u << 0;
constexpr uint32_t kStatusNaN = 1u << 1;

// One thread per (row, mask byte): 8 columns, two 4-groups or one 8-group.
template <int DT>
__device__ __forceinline__ uint32_t inf_code()
{
    return DT == NM_FP16 ? 0x7C00u : 0x7F80u;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void pack_check_kernel(const u32x4* __restrict__ W, const uint8_t* __restrict__ keep,
                                                            int64_t nbytes, int N, int M, uint32_t* __restrict__ status)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= nbytes)
        return;
    uint32_t bad = 0;
    if (keep) {
        const uint8_t* kp = keep + 8 * i;
        for (int g = 0; g < 8; g += M) {
            int cnt = 0;
            for (int j = 0; j < M; ++j)
                cnt += kp[g + j] != 0;
            if (cnt != N)
                bad |= kStatusBadMask;
        }
    } else {
        const u32x4 w = W[i];
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
        for (int d = 0; d < 4; ++d) {
            if ((words[d] & 0x7FFFu) > inf_code<DT>() || ((words[d] >> 16) & 0x7FFFu) > inf_code<DT>())
                bad |= kStatusNaN;
        }
    }
    if (bad)
        atomicOr(status, bad);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void pack_kernel(const u32x4* __restrict__ W, const uint8_t* __restrict__ keep,
                                                      int64_t nbytes, int N, int M, uint16_t* __restrict__ values,
                                                      uint8_t* __restrict__ masks)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= nbytes)
        return;
    const u32x4 wv = W[i];
    uint16_t w[8];
    w[0] = wv.x & 0xFFFF; w[1] = wv.x >> 16; w[2] = wv.y & 0xFFFF; w[3] = wv.y >> 16;
    w[4] = wv.z & 0xFFFF; w[5] = wv.z >> 16; w[6] = wv.w & 0xFFFF; w[7] = wv.w >> 16;
    uint32_t kb = 0;
    if (keep) {
        const uint8_t* kp = keep + 8 * i;
        for (int j = 0; j < 8; ++j)
            kb |= (uint32_t)(kp[j] != 0) << j;
    } else {
        // Column j is kept when fewer than N group members beat it: larger
        // magnitude, or equal magnitude at a lower column.  For non-NaN words
        // the unsigned order of (bits & 0x7FFF) is the order of |w|.
        for (int g = 0; g < 8; g += M) {
            for (int j = g; j < g + M; ++j) {
                const uint32_t mj = w[j] & 0x7FFFu;
                int beats = 0;
                for (int k = g; k < g + M; ++k) {
                    const uint32_t mk = w[k] & 0x7FFFu;
                    beats += (mk > mj) || (mk == mj && k < j);
                }
                kb |= (uint32_t)(beats < N) << j;
            }
        }
    }
    const int vpb = 8 / M * N;
    uint16_t* out = values + i * vpb;            // rows are whole bytes, so i * vpb is the fixed-step offset
    int k = 0;
    for (int j = 0; j < 8; ++j)
        if (((kb >> j) & 1u) && k < vpb)           // the check pass guarantees k < vpb; the guard keeps writes in bounds regardless
            out[k++] = w[j];
    masks[i] = (uint8_t)kb;
}

// ---- host side --------------------------------------------------------------

int g_rows_per_block_sparse = 0;   // 0 = built-in heuristic; NMSPMV_ROWS_PER_BLOCK overrides
std::once_flag g_env_once;

void read_env()
{
    if (const char* s = std::getenv("NMSPMV_ROWS_PER_BLOCK"))
        g_rows_per_block_sparse = std::atoi(s);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (na == 0 || nb == 0)
        return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// A pointer may be NULL only when its buffer is empty.
bool ptr_ok(const void* p, size_t bytes, uintptr_t align)
{
    if (bytes == 0)
        return true;
    return p != nullptr && aligned(p, align);
}

int check_dtype(int dtype) { return (dtype == NM_FP16 || dtype == NM_BF16) ? NM_OK : NM_ERR_UNSUPPORTED; }

int check_rk(int64_t R, int64_t K)
{
    if (R < 0 || K < 0 || R > INT32_MAX || K > INT32_MAX || K % 8 != 0)
        return NM_ERR_BAD_SHAPE;
    return NM_OK;
}

int check_nm(int64_t K, int N, int M)
{
    if ((M != 4 && M != 8) || N < 1 || N >= M || K % M != 0)
        return NM_ERR_BAD_SHAPE;
    return NM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? NM_OK : NM_ERR_HIP; }

int launch_zero(void* y, int64_t n, hipStream_t s)
{
    if (n == 0)
        return NM_OK;
    (void)hipGetLastError();
    const int64_t blocks = (n + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, (uint16_t*)y, n);
    return hip_status(hipGetLastError());
}

struct RowdotLaunch {
    int rows_per_block;
    int tile_cols;
    size_t lds_bytes;
    unsigned grid;
};

RowdotLaunch plan_rowdot(bool sparse, int64_t R, int64_t K, int B)
{
    std::call_once(g_env_once, read_env);
    RowdotLaunch L;
    // x tile: all of K when it fits, else the largest multiple of 1024 columns.
    int64_t tile = K;
    if ((int64_t)B * K * 2 > kXTileBudget)
        tile = ((int64_t)kXTileBudget / (2 * B)) / 1024 * 1024;
    L.tile_cols = (int)tile;
    int rpb = sparse ? g_rows_per_block_sparse : 0;
    if (rpb <= 0)
        rpb = 16;
    L.rows_per_block = rpb;
    const bool multi = tile < K;
    L.lds_bytes = (sparse ? 256 * sizeof(u32x4) : 0) + (size_t)B * tile * 2 + (multi ? (size_t)rpb * B * 4 : 0);
    L.grid = (unsigned)((R + rpb - 1) / rpb);
    return L;
}

template <bool SPARSE, int DT, int NB>
int launch_rowdot(const void* w, const void* m, const void* x, void* y, int R, int K, hipStream_t s)
{
    const RowdotLaunch L = plan_rowdot(SPARSE, R, K, NB);
    (void)hipGetLastError();
    hipLaunchKernelGGL((rowdot_kernel<SPARSE, DT, NB>), dim3(L.grid), dim3(kBlock), L.lds_bytes, s,
                       (const u32x4*)w, (const uint16_t*)m, (const u32x4*)x, (uint16_t*)y, R, K, L.rows_per_block,
                       L.tile_cols);
    return hip_status(hipGetLastError());
}

template <int DT, int NB>
int launch_generic(const void* v, const uint8_t* m, const void* x, void* y, int R, int K, int N, int M, hipStream_t s)
{
    (void)hipGetLastError();
    const unsigned grid = (unsigned)((R + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL((generic_spmv_kernel<DT, NB>), dim3(grid), dim3(kBlock), 0, s, (const uint16_t*)v, m,
                       (const uint16_t*)x, (uint16_t*)y, R, K, N, M);
    return hip_status(hipGetLastError());
}

template <template <int, int> class F, typename... A>
int dispatch(int dtype, int B, A... a)
{
    if (dtype == NM_FP16) {
        switch (B) {
        case 1: return F<NM_FP16, 1>::run(a...);
        case 2: return F<NM_FP16, 2>::run(a...);
        case 3: return F<NM_FP16, 3>::run(a...);
        case 4: return F<NM_FP16, 4>::run(a...);
        case 5: return F<NM_FP16, 5>::run(a...);
        case 6: return F<NM_FP16, 6>::run(a...);
        case 7: return F<NM_FP16, 7>::run(a...);
        case 8: return F<NM_FP16, 8>::run(a...);
        }
    } else {
        switch (B) {
        case 1: return F<NM_BF16, 1>::run(a...);
        case 2: return F<NM_BF16, 2>::run(a...);
        case 3: return F<NM_BF16, 3>::run(a...);
        case 4: return F<NM_BF16, 4>::run(a...);
        case 5: return F<NM_BF16, 5>::run(a...);
        case 6: return F<NM_BF16, 6>::run(a...);
        case 7: return F<NM_BF16, 7>::run(a...);
        case 8: return F<NM_BF16, 8>::run(a...);
        }
    }
    return NM_ERR_BAD_SHAPE;
}

template <int DT, int NB>
struct SparseFast {
    static int run(const void* v, const uint8_t* m, const void* x, void* y, int R, int K, hipStream_t s)
    {
        return launch_rowdot<true, DT, NB>(v, m, x, y, R, K, s);
    }
};

template <int DT, int NB>
struct SparseGeneric {
    static int run(const void* v, const uint8_t* m, const void* x, void* y, int R, int K, int N, int M, hipStream_t s)
    {
        return launch_generic<DT, NB>(v, m, x, y, R, K, N, M, s);
    }
};

template <int DT, int NB>
struct Dense {
    static int run(const void* w, const void* x, void* y, int R, int K, hipStream_t s)
    {
        return launch_rowdot<false, DT, NB>(w, nullptr, x, y, R, K, s);
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

}  // namespace

extern "C" {

int nm_version(void) { return 100; }

const char* nm_status_string(int status)
{
    switch (status) {
    case NM_OK: return "NM_OK";
    case NM_ERR_INVALID_ARG: return "NM_ERR_INVALID_ARG";
    case NM_ERR_BAD_SHAPE: return "NM_ERR_BAD_SHAPE";
    case NM_ERR_UNSUPPORTED: return "NM_ERR_UNSUPPORTED";
    case NM_ERR_BAD_MASK: return "NM_ERR_BAD_MASK";
    case NM_ERR_NONFINITE: return "NM_ERR_NONFINITE";
    case NM_ERR_HIP: return "NM_ERR_HIP";
    default: return "NM_ERR_UNKNOWN";
    }
}

int nm_spmv(const void* values, const uint8_t* masks, int64_t R, int64_t K, int N, int M, int dtype, const void* x,
            int B, void* y, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK || (st = check_nm(K, N, M)) != NM_OK)
        return st;
    if (B < 1 || B > 8)
        return NM_ERR_BAD_SHAPE;
    const size_t vbytes = (size_t)R * (size_t)(K / M * N) * 2, mbytes = (size_t)R * (size_t)(K / 8);
    const size_t xbytes = (size_t)B * (size_t)K * 2, ybytes = (size_t)B * (size_t)R * 2;
    if (!ptr_ok(values, vbytes, 16) || !ptr_ok(masks, mbytes, 16) || !ptr_ok(x, xbytes, 16) || !ptr_ok(y, ybytes, 2))
        return NM_ERR_INVALID_ARG;
    if (overlaps(y, ybytes, values, vbytes) || overlaps(y, ybytes, masks, mbytes) || overlaps(y, ybytes, x, xbytes))
        return NM_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (R == 0)
        return NM_OK;
    if (K == 0)
        return launch_zero(y, (int64_t)B * R, s);
    if (2 * N == M && K % 16 == 0)
        return dispatch<SparseFast>(dtype, B, values, masks, x, y, (int)R, (int)K, s);
    return dispatch<SparseGeneric>(dtype, B, values, masks, x, y, (int)R, (int)K, N, M, s);
}

int nm_gemv_dense(const void* W, int64_t R, int64_t K, int dtype, const void* x, int B, void* y, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK)
        return st;
    if (B < 1 || B > 8)
        return NM_ERR_BAD_SHAPE;
    const size_t wbytes = (size_t)R * (size_t)K * 2, xbytes = (size_t)B * (size_t)K * 2, ybytes = (size_t)B * (size_t)R * 2;
    if (!ptr_ok(W, wbytes, 16) || !ptr_ok(x, xbytes, 16) || !ptr_ok(y, ybytes, 2))
        return NM_ERR_INVALID_ARG;
    if (overlaps(y, ybytes, W, wbytes) || overlaps(y, ybytes, x, xbytes))
        return NM_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (R == 0)
        return NM_OK;
    if (K == 0)
        return launch_zero(y, (int64_t)B * R, s);
    return dispatch<Dense>(dtype, B, W, x, y, (int)R, (int)K, s);
}

int nm_pack(const void* W, const uint8_t* keep, int64_t R, int64_t K, int N, int M, int dtype, void* values,
            uint8_t* masks, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK || (st = check_nm(K, N, M)) != NM_OK)
        return st;
    const size_t wbytes = (size_t)R * (size_t)K * 2, kbytes = keep ? (size_t)R * (size_t)K : 0;
    const size_t vbytes = (size_t)R * (size_t)(K / M * N) * 2, mbytes = (size_t)R * (size_t)(K / 8);
    if (!ptr_ok(W, wbytes, 16) || !ptr_ok(values, vbytes, 16) || !ptr_ok(masks, mbytes, 16))
        return NM_ERR_INVALID_ARG;
    if (overlaps(values, vbytes, W, wbytes) || overlaps(values, vbytes, keep, kbytes) ||
        overlaps(masks, mbytes, W, wbytes) || overlaps(masks, mbytes, keep, kbytes) ||
        overlaps(values, vbytes, masks, mbytes))
        return NM_ERR_INVALID_ARG;
    const int64_t nbytes = R * (K / 8);
    if (nbytes == 0)
        return NM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_pack_mutex);
    uint32_t* status = nullptr;
    if ((st = status_word(&status)) != NM_OK)
        return st;
    const unsigned grid = (unsigned)((nbytes + kBlock - 1) / kBlock);
    (void)hipGetLastError();
    if (hipMemsetAsync(status, 0, sizeof(uint32_t), s) != hipSuccess)
        return NM_ERR_HIP;
    if (dtype == NM_FP16)
        hipLaunchKernelGGL(pack_check_kernel<NM_FP16>, dim3(grid), dim3(kBlock), 0, s, (const u32x4*)W, keep, nbytes,
                           N, M, status);
    else
        hipLaunchKernelGGL(pack_check_kernel<NM_BF16>, dim3(grid), dim3(kBlock), 0, s, (const u32x4*)W, keep, nbytes,
                           N, M, status);
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
    if (dtype == NM_FP16)
        hipLaunchKernelGGL(pack_kernel<NM_FP16>, dim3(grid), dim3(kBlock), 0, s, (const u32x4*)W, keep, nbytes, N, M,
                           (uint16_t*)values, masks);
    else
        hipLaunchKernelGGL(pack_kernel<NM_BF16>, dim3(grid), dim3(kBlock), 0, s, (const u32x4*)W, keep, nbytes, N, M,
                           (uint16_t*)values, masks);
    if (hipGetLastError() != hipSuccess)
        return NM_ERR_HIP;
    return hip_status(hipStreamSynchronize(s));
}

}  // extern "C"
