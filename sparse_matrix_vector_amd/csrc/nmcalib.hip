// nmcalib.hip -- decoding-aware calibration for libnmspmv (gfx950).
//
// SparseDecoding builds its pruning objective from the inputs a layer sees
// while the dense model generates token by token, the prefill excluded, and
// guides pruning with the Hessian of that objective ("SparseDecoding:
// Decoding-Aware Pruning for Accurate and Efficient LLM Inference", Abstract;
// "SparseDecoding Makes LLM Pruning Aware of Generation", Key points and the
// section on why fixed-text calibration misses).  The pages give no formula;
// this file implements the plainest reading:
//   * nm_calib_accumulate: H += sum over decode rows t of x_t x_t^T, the
//     Hessian (up to a constant) of a linear layer's squared output error;
//   * nm_calib_keep_mask: per M-group keep the N columns of largest saliency
//     w^2 H_jj (the optimal-brain-surgeon saliency with H taken diagonal),
//     lower column on ties, as a keep-mask for nm_pack.
//
// The accumulation is a dense contraction over the token axis, so it runs on
// the matrix cores: v_mfma_f32_32x32x16 (fp16 / bf16 in, fp32 out), one
// 128 x 128 tile of the upper triangle of H per 256-thread block (added to
// its mirror tile too), 64 token rows per step staged in LDS column by column.
// Its traffic is H's read and write (8 K^2 bytes).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nm_decode.h"
#include "nmspmv.h"

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 128;        // H tile per block (rows i and columns j)
constexpr int kTT = 64;           // token rows per staging step
constexpr int kTPitch = kTT + 8;  // LDS halves per staged column: 16-byte reads of 16 columns hit distinct banks
constexpr int kTW = kTT / 4;      // token rows per wave per step
constexpr int kMPitch = 64 + 1;   // floats per row of a wave's transposed half-quarter (mirror tile)
static_assert(4 * 32 * kMPitch * 4 <= 2 * kTile * kTPitch * 2, "mirror staging fits in the X staging area");

// ---- H += X_d^T X_d --------------------------------------------------------------

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// v_mfma_f32_32x32x16 (gfx950): lane l supplies 8 k-values of row l % 32 of A
// and of column l % 32 of B (A and B assign k to lanes and registers the same
// way), and holds D[i][j] for j = l % 32, i = 8 (v / 4) + 4 (l / 32) + v % 4 in
// accumulator v.  Here A = X^T (i, t) and B = X (t, j): both fragments are 8
// tokens of one column, and lane half h = l / 32 takes tokens 8 h .. 8 h + 7
// of the 16-token step, so the sum runs over exactly those tokens whatever
// order the hardware gives k inside the instruction.
template <int DT>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 acc)
{
    if constexpr (DT == NM_FP16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0, 0,
                                                      0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                       0, 0, 0);
}

// H is symmetric, so a block computes one tile S = X_I^T X_J of the upper
// triangle (bi <= bj, tiles numbered column by column) and adds it to both
// H[I][J] and, off the diagonal, H[J][I] (as S^T): half the matrix-core work
// and half the re-reads of X of covering every tile.
__device__ __forceinline__ void tile_of(int id, int& bi, int& bj)
{
    int c = (int)((sqrtf(8.f * (float)id + 1.f) - 1.f) * 0.5f);
    while ((c + 1) * (c + 2) / 2 <= id)
        ++c;
    while (c * (c + 1) / 2 > id)
        --c;
    bj = c;
    bi = id - c * (c + 1) / 2;
}

// Block id -> tile (bi, bj) owns S = X[:, 128 bi .. +128]^T X[:, 128 bj ..
// +128]; wave w owns the 64 x 64 quarter (w / 2, w % 2) as 2 x 2 matrix-core
// blocks.  The registers stay few enough for three blocks per CU (at
// K = 4096, all 528 tiles resident at once), so H is read only after the
// token loop, when the other blocks' loops overlap it.
// Each step stages 64 token rows of X's two column ranges in LDS transposed,
// [column][token], so that an operand (8 tokens of a column) is one 16-byte
// read: wave w loads tokens 16 w .. 16 w + 15, lanes 0-31 four columns of the
// I range and lanes 32-63 four of the J range (8-byte loads, 256 contiguous
// bytes per token row per half-wave), transposes them in registers with byte
// permutes and writes two 16-byte runs per column.  The next step's loads are
// in flight while a step is multiplied; every load is issued whatever the
// token count (tokens past T reload row 0 and are zeroed when staged), so
// that the compiler waits for exactly the step it stages.  The decode flags
// ride with the loads (lane l of a wave fetches its token l % 16) and are
// read across the wave when staged.  Tokens past T, prefill tokens and
// columns past K are zero.
// Off the diagonal, S^T is added into H[J][I] through LDS, 32 rows of a
// wave's quarter at a time, so that each H row is read and written as 64
// consecutive floats.
template <int DT>
__global__ __launch_bounds__(256, 3) void calib_accumulate_kernel(const uint16_t* __restrict__ X,
                                                               const uint8_t* __restrict__ decode, int T, int K,
                                                               float* __restrict__ H)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[2 * kTile * kTPitch];   // [range][column][token]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bi, bj;
    tile_of(blockIdx.x, bi, bj);
    const int i0 = bi * kTile, j0 = bj * kTile;
    const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;

    f32x16 acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[m][n][v] = 0.f;

    // Staging role: range r (0: columns I, 1: J), columns c4 .. c4 + 3 of it,
    // tokens kTW wave .. kTW wave + kTW - 1 of the step.
    const int r = lane >> 5, c4 = 4 * (lane & 31);
    const int col = (r == 0 ? i0 : j0) + c4;
    const bool col_ok = col < K;                   // K % 4 == 0: four columns in or out together
    const uint32_t loff = 2u * (uint32_t)(col_ok ? col : 0);   // the lane's byte offset in a token row
    const uint8_t* flags = decode ? decode : reinterpret_cast<const uint8_t*>(X);   // (read, then ignored)
    struct Step {
        u32x2 w[kTW];
        uint32_t f;                                // decode flag of token (lane % kTW) of the wave's rows
    };
    auto load_step = [&](Step& st, int t0) {
#pragma unroll
        for (int e = 0; e < kTW; ++e) {
            const int t = t0 + kTW * wave + e;  // wave-uniform: a scalar row base plus the lane's offset
            const char* row = reinterpret_cast<const char*>(X) + (size_t)(t < T ? t : 0) * K * 2;
            st.w[e] = *reinterpret_cast<const u32x2*>(row + loff);
        }
        const int tf = t0 + kTW * wave + (lane & (kTW - 1));
        st.f = flags[tf < T ? tf : 0];
    };
    auto store_step = [&](const Step& st, int t0) {
        uint32_t w[kTW][2];
#pragma unroll
        for (int e = 0; e < kTW; ++e) {
            const int t = t0 + kTW * wave + e;
            const bool live = col_ok && t < T && (!decode || __builtin_amdgcn_readlane((int)st.f, e) != 0);
            w[e][0] = live ? st.w[e].x : 0u;
            w[e][1] = live ? st.w[e].y : 0u;
        }
        // Column c4 + u (u = 0..3) takes half u % 2 of word u / 2 of each token.
#pragma unroll
        for (int g = 0; g < kTW / 8; ++g)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;   // high or low halves of two words
                const uint32_t(*wg)[2] = w + 8 * g;
                u32x4 o;
                o.x = __builtin_amdgcn_perm(wg[1][u >> 1], wg[0][u >> 1], sel);
                o.y = __builtin_amdgcn_perm(wg[3][u >> 1], wg[2][u >> 1], sel);
                o.z = __builtin_amdgcn_perm(wg[5][u >> 1], wg[4][u >> 1], sel);
                o.w = __builtin_amdgcn_perm(wg[7][u >> 1], wg[6][u >> 1], sel);
                *reinterpret_cast<u32x4*>(&xs[(r * kTile + c4 + u) * kTPitch + kTW * wave + 8 * g]) = o;
            }
    };
    auto multiply = [&]() {
#pragma unroll
        for (int k = 0; k < kTT / 16; ++k) {
            const int tk = 16 * k + 8 * (lane >> 5);
            u32x4 a[2], b[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                a[m] = *reinterpret_cast<const u32x4*>(&xs[(wi + 32 * m + (lane & 31)) * kTPitch + tk]);
                b[m] = *reinterpret_cast<const u32x4*>(&xs[(kTile + wj + 32 * m + (lane & 31)) * kTPitch + tk]);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[m][n] = mfma<DT>(a[m], b[n], acc[m][n]);
        }
    };

    Step st;
    load_step(st, 0);
    for (int t0 = 0; t0 < T; t0 += kTT) {
        __syncthreads();                          // the previous step's tiles are no longer read
        store_step(st, t0);
        __syncthreads();
        load_step(st, t0 + kTT);                  // in flight during this step's products
        multiply();
    }
    // H[I][J] += the block's sums, one 32-row half of the wave's quarter at a
    // time (its 32 values read, then written: 32 consecutive columns per
    // half-wave), addressed from the tile's corner.
    float* const Ht = H + (size_t)i0 * K + j0;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float h[2][16];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int jl = wj + 32 * n + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int il = wi + 32 * m + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                h[n][v] = (i0 + il < K && j0 + jl < K) ? Ht[(uint32_t)(il * K + jl)] : 0.f;
            }
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int jl = wj + 32 * n + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int il = wi + 32 * m + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (i0 + il < K && j0 + jl < K)
                    Ht[(uint32_t)(il * K + jl)] = h[n][v] + acc[m][n][v];
            }
        }
    }
    if (bi == bj)
        return;
    // H[J][I] += S^T: rows j = 32 n + (lane % 32) of the wave's quarter go to
    // LDS as tq[j][i], then each of those 32 H rows is updated by all 64 lanes.
    float* tq = reinterpret_cast<float*>(xs) + wave * 32 * kMPitch;
    float* const Hm = H + (size_t)j0 * K + i0;   // the mirror tile's corner
    const int ci = i0 + wi + lane;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        __syncthreads();                          // xs (or the previous half) is no longer read
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                tq[(lane & 31) * kMPitch + 32 * m + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)] = acc[m][n][v];
        __syncthreads();
        float h[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const int jl = wj + 32 * n + e;
            h[e] = (j0 + jl < K && ci < K) ? Hm[(uint32_t)(jl * K + wi + lane)] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const int jl = wj + 32 * n + e;
            if (j0 + jl < K && ci < K)
                Hm[(uint32_t)(jl * K + wi + lane)] = h[e] + tq[e * kMPitch + lane];
        }
    }
}

// ---- saliency keep-mask -----------------------------------------------------------

// One thread per (row, 8 columns): two 4-groups or one 8-group.  Saliency
// w^2 h is exact in double (w^2 has at most 22 significant bits, h 24); a NaN
// saliency ranks below every other.  Column j is kept when fewer than N group
// members beat it: larger saliency, or equal saliency at a lower column.
template <int DT>
__global__ __launch_bounds__(256) void calib_keep_kernel(const u32x4* __restrict__ W, const float* __restrict__ h,
                                                         int64_t h_stride, int64_t nunits, int64_t units_per_row, int N,
                                                         int M, u32x2* __restrict__ keep)
{
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= nunits)
        return;
    const int64_t c0 = (u % units_per_row) * 8;
    const u32x4 wv = W[u];
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
    double s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double w = nm_decode::w_to_f64<DT>((words[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        const double hv = nm_decode::f32_to_f64(h[(c0 + e) * h_stride]);
        const double v = w * w * hv;
        s[e] = v != v ? -1.0 : v;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int g = e / M * M;
        int beats = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k >= g && k < g + M)
                beats += (s[k] > s[e]) || (s[k] == s[e] && k < e);
        const uint32_t bit = beats < N ? 1u : 0u;
        if (e < 4)
            lo |= bit << (8 * e);
        else
            hi |= bit << (8 * (e - 4));
    }
    keep[u] = u32x2{lo, hi};
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (na == 0 || nb == 0 || !a || !b)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

bool ptr_ok(const void* p, size_t bytes, uintptr_t align)
{
    if (bytes == 0)
        return true;
    return p != nullptr && (reinterpret_cast<uintptr_t>(p) & (align - 1)) == 0;
}

int launched() { return hipGetLastError() == hipSuccess ? NM_OK : NM_ERR_HIP; }

}  // namespace

extern "C" {

int nm_calib_accumulate(const void* X, const uint8_t* decode, int64_t T, int64_t K, int dtype, float* H, void* stream)
{
    if (dtype != NM_FP16 && dtype != NM_BF16)
        return NM_ERR_UNSUPPORTED;
    if (T < 0 || K < 0 || K % 8 != 0 || T > INT32_MAX || K > 65536)
        return NM_ERR_BAD_SHAPE;
    const size_t xbytes = (size_t)T * (size_t)K * 2, hbytes = (size_t)K * (size_t)K * 4;
    if (!ptr_ok(X, xbytes, 16) || !ptr_ok(H, hbytes, 4))
        return NM_ERR_INVALID_ARG;
    if (overlaps(H, hbytes, X, xbytes) || overlaps(H, hbytes, decode, (size_t)T))
        return NM_ERR_INVALID_ARG;
    if (T == 0 || K == 0)
        return NM_OK;
    const unsigned nb = (unsigned)((K + kTile - 1) / kTile);
    const unsigned tiles = nb * (nb + 1) / 2;     // upper triangle, diagonal included
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (dtype == NM_FP16)
        hipLaunchKernelGGL(calib_accumulate_kernel<NM_FP16>, dim3(tiles), dim3(256), 0, s,
                           static_cast<const uint16_t*>(X), decode, (int)T, (int)K, H);
    else
        hipLaunchKernelGGL(calib_accumulate_kernel<NM_BF16>, dim3(tiles), dim3(256), 0, s,
                           static_cast<const uint16_t*>(X), decode, (int)T, (int)K, H);
    return launched();
}

int nm_calib_keep_mask(const void* W, const float* h, int64_t h_stride, int64_t R, int64_t K, int N, int M, int dtype,
                       uint8_t* keep, void* stream)
{
    if (dtype != NM_FP16 && dtype != NM_BF16)
        return NM_ERR_UNSUPPORTED;
    if (R < 0 || K < 0 || K % 8 != 0 || (M != 4 && M != 8) || N < 1 || N >= M || K % M != 0 || h_stride < 1)
        return NM_ERR_BAD_SHAPE;
    const size_t wbytes = (size_t)R * (size_t)K * 2, kbytes = (size_t)R * (size_t)K;
    const size_t hbytes = K > 0 ? ((size_t)(K - 1) * (size_t)h_stride + 1) * 4 : 0;
    if (!ptr_ok(W, wbytes, 16) || !ptr_ok(keep, kbytes, 8) || !ptr_ok(h, hbytes, 4))
        return NM_ERR_INVALID_ARG;
    if (overlaps(keep, kbytes, W, wbytes) || overlaps(keep, kbytes, h, hbytes))
        return NM_ERR_INVALID_ARG;
    const int64_t nunits = R * (K / 8);
    if (nunits == 0)
        return NM_OK;
    const unsigned grid = (unsigned)((nunits + 255) / 256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (dtype == NM_FP16)
        hipLaunchKernelGGL(calib_keep_kernel<NM_FP16>, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(W), h,
                           h_stride, nunits, K / 8, N, M, reinterpret_cast<u32x2*>(keep));
    else
        hipLaunchKernelGGL(calib_keep_kernel<NM_BF16>, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(W), h,
                           h_stride, nunits, K / 8, N, M, reinterpret_cast<u32x2*>(keep));
    return launched();
}

}  // extern "C"
