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
// the matrix cores: v_mfma_f32_32x32x8 (fp16 / bf16 in, fp32 out), 128 x 128
// tiles of H per 256-thread block, 32 token rows per step staged in LDS.
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
constexpr int kTT = 32;           // token rows per staging step
constexpr int kPitch = kTile + 8; // LDS row pitch in halves: rows t and t + 4 land 16 banks apart

// ---- H += X_d^T X_d --------------------------------------------------------------

// v_mfma_f32_32x32x8 operand layout (one block): lane l holds A[l % 32][4 (l / 32) + e]
// and B[4 (l / 32) + e][l % 32], e = 0..3, and the result D[i][j] for j = l % 32,
// i = 8 (v / 4) + 4 (l / 32) + v % 4 in accumulator v.  Here A = X^T (i, t) and
// B = X (t, j), so both fragments are 4 tokens of one column.
template <int DT>
__device__ __forceinline__ f32x16 mfma(u32x2 a, u32x2 b, f32x16 acc)
{
    if constexpr (DT == NM_FP16)
        return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), acc, 0, 0,
                                                    0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), acc,
                                                        0, 0, 0);
}

// Tokens t .. t + 3 of column c of a staged tile [token][column], packed in
// token order (lanes 0-31 read 32 consecutive columns: no bank conflicts).
__device__ __forceinline__ u32x2 frag(const uint16_t* tile, int t, int c)
{
    const uint32_t v0 = tile[t * kPitch + c], v1 = tile[(t + 1) * kPitch + c];
    const uint32_t v2 = tile[(t + 2) * kPitch + c], v3 = tile[(t + 3) * kPitch + c];
    return u32x2{v0 | (v1 << 16), v2 | (v3 << 16)};
}

// Block (bj, bi) owns H[128 bi .. +128][128 bj .. +128]; wave w owns the 64 x 64
// quarter (w / 2, w % 2) as 2 x 2 MFMA blocks.  Each step stages 32 token rows
// of X's two column ranges, zeroing rows past T and prefill rows.
template <int DT>
__global__ __launch_bounds__(256) void calib_accumulate_kernel(const uint16_t* __restrict__ X,
                                                               const uint8_t* __restrict__ decode, int T, int K,
                                                               float* __restrict__ H)
{
    __shared__ __attribute__((aligned(16))) uint16_t xi[kTT * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t xj[kTT * kPitch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
    const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[a][b][v] = 0.f;

    // Staging: thread -> token row tt = tid / 8 and 16 columns 16 q .. 16 q + 15
    // (q = tid % 8) of each range: two 16-byte loads and stores per range.
    const int tt = tid >> 3, q = tid & 7;
    for (int t0 = 0; t0 < T; t0 += kTT) {
        const int t = t0 + tt;
        const bool live = t < T && (!decode || decode[t]);
        u32x4 vi[2], vj[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ci = i0 + 16 * q + 8 * h, cj = j0 + 16 * q + 8 * h;
            const u32x4 z = {0u, 0u, 0u, 0u};
            vi[h] = live && ci < K ? *reinterpret_cast<const u32x4*>(X + (size_t)t * K + ci) : z;
            vj[h] = live && cj < K ? *reinterpret_cast<const u32x4*>(X + (size_t)t * K + cj) : z;
        }
        __syncthreads();                          // the previous step's tiles are no longer read
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<u32x4*>(&xi[tt * kPitch + 16 * q + 8 * h]) = vi[h];
            *reinterpret_cast<u32x4*>(&xj[tt * kPitch + 16 * q + 8 * h]) = vj[h];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kTT / 8; ++k) {
            const int tk = 8 * k + 4 * (lane >> 5);
            u32x2 a[2], b[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                a[m] = frag(xi, tk, wi + 32 * m + (lane & 31));
                b[m] = frag(xj, tk, wj + 32 * m + (lane & 31));
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[m][n] = mfma<DT>(a[m], b[n], acc[m][n]);
        }
    }
    // H += the block's sums (32 consecutive columns per half-wave: coalesced).
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int j = j0 + wj + 32 * n + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = i0 + wi + 32 * m + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (i < K && j < K)
                    H[(size_t)i * K + j] += acc[m][n][v];
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (dtype == NM_FP16)
        hipLaunchKernelGGL(calib_accumulate_kernel<NM_FP16>, dim3(nb, nb), dim3(256), 0, s,
                           static_cast<const uint16_t*>(X), decode, (int)T, (int)K, H);
    else
        hipLaunchKernelGGL(calib_accumulate_kernel<NM_BF16>, dim3(nb, nb), dim3(256), 0, s,
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
