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
// its mirror tile too), X streamed into an LDS ring by global-to-LDS loads
// and read back transposed (ds_read_b64_tr_b16).
// Its traffic is H's read and write (8 K^2 bytes).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "nm_decode.h"
#include "nm_launch.h"
#include "nmspmv.h"

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 128;        // H tile per block (rows i and columns j)
constexpr int kTS = 32;           // token rows per stage
constexpr int kSlots = 3;         // stages in the block's LDS ring
constexpr int kRowBytes = kTile * 2;                    // one token row of one column range
constexpr int kRangeBytes = kTS * kRowBytes;            // 8 KB
constexpr int kFlagBytes = 4 * 256;                     // each wave's 64 decode-flag dwords
constexpr int kSlotBytes = 2 * kRangeBytes + kFlagBytes;
constexpr int kMPitch = 64 + 1;   // floats per row of a wave's transposed half-quarter (mirror tile)
constexpr int kMirrorBytes = 4 * 32 * kMPitch * 4;
static_assert(kMirrorBytes <= kSlots * kSlotBytes, "the mirror staging fits in the ring");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;

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

// Global-to-LDS loads into the kernel's dynamic LDS (which starts at offset
// 0): 16 bytes per lane to lds_offset + 16 lane, or one byte per lane,
// zero-extended, to lds_offset + 4 lane (lds_offset wave-uniform).  The LDS
// side is addressed by offset, not through the array the kernel reads, so
// the compiler does not wait for these loads before every LDS read; the
// kernel's own waits and barriers order them.
template <int BYTES>
__device__ __forceinline__ void dma(const void* g, uint32_t lds_offset)
{
    static_assert(BYTES == 16 || BYTES == 1, "16- or 1-byte lanes");
#if defined(__HIP_DEVICE_COMPILE__)
    lds_void_t* dst = (lds_void_t*)((lds_u8_t*)nullptr + lds_offset);
    if constexpr (BYTES == 16)
        __builtin_amdgcn_global_load_lds(g, dst, 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(g, dst, 1, 0, 0);
#else
    (void)g;
    (void)lds_offset;
#endif
}

// s_waitcnt with vmcnt <= N and the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Position of 16-byte column unit u in token row t (0..31) of a staged range:
// u ^ swz(t), so that the operand reads below, four rows by four units per
// half-wave, fall in distinct banks.
__device__ __forceinline__ int swz(int t) { return 4 * ((t + (t >> 3)) & 3); }

// LDS byte address of the 8 bytes lane `lane` hands to transposing read s of
// the operand "8 tokens (tb .. tb + 7 of the stage) of column c0 + l % 32 of
// the range at rng" for lane l.  In a group of 16 lanes, ds_read_b64_tr_b16
// gives lane i half (i % 4) of the 8 bytes that lane 4 e + i / 4 addresses,
// as its element e; so lane j addresses token tb + 4 s + j / 4, columns
// c0 + 4 (j % 4) .. + 3, and lane i receives 4 tokens of column c0 + i.
__device__ __forceinline__ uint32_t operand_addr(uint32_t rng, int c0, int tb, int lane, int s)
{
    const int g = lane >> 4, j = lane & 15;
    const int cb = c0 + 16 * (g & 1), t = tb + 8 * (g >> 1) + (j >> 2) + 4 * s;
    const int u = cb / 8 + ((j & 3) >> 1);
    return rng + (uint32_t)(t * kRowBytes + ((u ^ swz(t)) * 16) + 8 * (j & 1));
}

// The four operands of one 16-token matrix-core step (a[m]: range I, columns
// wi + 32 m; b[m]: range J, columns wj + 32 m), eight transposing reads.
// They are issued in one asm block that waits for them itself: the compiler
// knows nothing of what the builtin form reads and would otherwise wait for
// every global-to-LDS load in flight before each read.
__device__ __forceinline__ void step_operands(uint32_t slot, int wi, int wj, int tb, int lane, u32x4* a, u32x4* b)
{
    uint32_t ad[8];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            ad[2 * m + s] = operand_addr(slot, wi + 32 * m, tb, lane, s);
            ad[4 + 2 * m + s] = operand_addr(slot + kRangeBytes, wj + 32 * m, tb, lane, s);
        }
    u32x2 r[8];
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
#else
    for (int i = 0; i < 8; ++i)
        r[i] = u32x2{ad[i], 0u};
#endif
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        a[m] = u32x4{r[2 * m].x, r[2 * m].y, r[2 * m + 1].x, r[2 * m + 1].y};
        b[m] = u32x4{r[4 + 2 * m].x, r[4 + 2 * m].y, r[4 + 2 * m + 1].x, r[4 + 2 * m + 1].y};
    }
}

// Block id -> tile (bi, bj) owns S = X[:, 128 bi .. +128]^T X[:, 128 bj ..
// +128]; wave w owns the 64 x 64 quarter (w / 2, w % 2) as 2 x 2 matrix-core
// blocks.
// X goes from HBM/L2 straight into a three-slot LDS ring of 32-token stages,
// untransposed ([range][token][128 columns], column units swizzled by row),
// with global-to-LDS loads: per stage each wave issues four 1 KB loads (four
// token rows of one range; 16 lanes per row) and one 64-byte load of the
// stage's decode flags into its own corner of the slot, so every stage costs
// each wave the same five loads and the waits are fixed counts.  Per stage a
// wave waits for its own loads, meets the block at a barrier (no memory
// fence: the wait already covers its loads into LDS), issues the loads of
// the stage after next into the slot every wave has just finished reading,
// and multiplies: operands come from transposing LDS reads, no register
// staging.  Loads are issued whatever T is (tokens past T reload row T - 1;
// columns past K reload column 0 and only reach entries never stored), and
// tokens past T or flagged prefill are zeroed in both operands from a
// wave-uniform bit word, so non-finite prefill rows cannot leak in.
// Then H[I][J] += S, and off the diagonal H[J][I] += S^T through LDS, 32 rows
// of a wave's quarter at a time, so that each H row is read and written as 64
// consecutive floats.
template <int DT>
__global__ __launch_bounds__(256, 3) void calib_accumulate_kernel(const uint16_t* __restrict__ X,
                                                                  const uint8_t* __restrict__ decode, int T, int K,
                                                                  float* __restrict__ H)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // kSlots * kSlotBytes, at LDS offset 0
    lds_u8_t* const L = (lds_u8_t*)smem;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bi, bj;
    tile_of(blockIdx.x, bi, bj);
    const int i0 = bi * kTile, j0 = bj * kTile;
    const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;

    // Load role: instruction q of the wave is n = wave + 4 q: range n / 8,
    // token rows 4 (n % 8) .. + 3; the lane takes row lane / 16 of them and
    // LDS position lane % 16, i.e. column unit (lane % 16) ^ swz(row).
    int scol[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = wave + 4 * q, r = n >> 3, t = 4 * (n & 7) + (lane >> 4);
        const int col = (r == 0 ? i0 : j0) + 8 * ((lane & 15) ^ swz(t));
        scol[q] = col < K ? col : 0;             // K % 8 == 0: a unit is in or out whole
    }
    const uint8_t* flags = decode ? decode : reinterpret_cast<const uint8_t*>(X);   // (read, then ignored)
    auto issue = [&](int st) {
        const int t0 = st * kTS;
        const uint32_t slot = (uint32_t)((st % kSlots) * kSlotBytes);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = wave + 4 * q;
            const int tok = min(t0 + 4 * (n & 7) + (lane >> 4), T - 1);
            dma<16>(X + (size_t)tok * K + scol[q], slot + (n >> 3) * kRangeBytes + (n & 7) * 1024);
        }
        dma<1>(flags + min(t0 + lane, T - 1), slot + 2 * kRangeBytes + wave * 256);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[m][n][v] = 0.f;

    auto consume = [&](int st) {
        const int t0 = st * kTS;
        const uint32_t slot = (uint32_t)((st % kSlots) * kSlotBytes);
        const uint32_t fd = *(const lds_u32_t*)(L + slot + 2 * kRangeBytes + wave * 256 + (lane & 31) * 4);
        const bool ok = t0 + (lane & 31) < T && (!decode || fd != 0u);
        const uint32_t fw = (uint32_t)__builtin_amdgcn_ballot_w64(ok);   // bit e: token t0 + e enters H
#pragma unroll
        for (int k = 0; k < kTS / 16; ++k) {
            u32x4 a[2], b[2];
            step_operands(slot, wi, wj, 16 * k, lane, a, b);
            if (fw != 0xFFFFFFFFu) {
                const uint32_t bits = (fw >> (16 * k + 8 * (lane >> 5))) & 0xFFu;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t mk = ((bits >> (2 * d)) & 1u ? 0x0000FFFFu : 0u) |
                                        ((bits >> (2 * d + 1)) & 1u ? 0xFFFF0000u : 0u);
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        a[m][d] &= mk;
                        b[m][d] &= mk;
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[m][n] = mfma<DT>(a[m], b[n], acc[m][n]);
        }
    };

    const int nst = (T + kTS - 1) / kTS;
    issue(0);
    issue(1);
    for (int st = 0; st < nst; ++st) {
        wait_vmcnt<5>();                          // this wave's loads of stage st have landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();             // every wave's have; all finished reading stage st - 1
        asm volatile("" ::: "memory");
        issue(st + 2);                            // into stage st - 1's slot
        consume(st);
    }
    wait_vmcnt<0>();                              // the ring's last loads (past T) have landed
    __syncthreads();                              // and every wave is done with the ring

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
    float* tq = reinterpret_cast<float*>(smem) + wave * 32 * kMPitch;
    float* const Hm = H + (size_t)j0 * K + i0;   // the mirror tile's corner
    const int ci = i0 + wi + lane;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        __syncthreads();                          // the previous half is no longer read
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
// saliency ranks below every number, -inf included, and NaNs rank equal.
// Column j is kept when fewer than N group members beat it: a higher rank,
// or an equal one at a lower column.
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
        s[e] = v;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int g = e / M * M;
        int beats = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k >= g && k < g + M)
                beats += (s[k] == s[k] && (s[e] != s[e] || s[k] > s[e])) ||
                         (((s[k] != s[k]) ? (s[e] != s[e]) : (s[k] == s[e])) && k < e);
        const uint32_t bit = beats < N ? 1u : 0u;
        if (e < 4)
            lo |= bit << (8 * e);
        else
            hi |= bit << (8 * (e - 4));
    }
    keep[u] = u32x2{lo, hi};
}

int launched() { return hipGetLastError() == hipSuccess ? NM_OK : NM_ERR_HIP; }

}  // namespace

// ---- the kernel side of the entry points (arguments checked by nmapi.cpp) --------

int nmk::calib_accumulate(const void* X, const uint8_t* decode, int64_t T, int64_t K, int dtype, float* H,
                          void* stream)
{
    const unsigned nb = (unsigned)((K + kTile - 1) / kTile);
    const unsigned tiles = nb * (nb + 1) / 2;     // upper triangle, diagonal included
    hipStream_t s = static_cast<hipStream_t>(stream);
    // At most 2^30 rows per launch, so that the kernel's token arithmetic
    // (which runs two 32-row stages past its rows) stays in 32 bits; the
    // launches add into H one after another.
    constexpr int64_t kMaxRows = int64_t(1) << 30;
    for (int64_t t0 = 0; t0 < T; t0 += kMaxRows) {
        const int Tc = (int)std::min<int64_t>(kMaxRows, T - t0);
        const uint16_t* Xc = static_cast<const uint16_t*>(X) + t0 * K;
        const uint8_t* dc = decode ? decode + t0 : nullptr;
        (void)hipGetLastError();
        if (dtype == NM_FP16)
            hipLaunchKernelGGL(calib_accumulate_kernel<NM_FP16>, dim3(tiles), dim3(256), kSlots * kSlotBytes, s, Xc,
                               dc, Tc, (int)K, H);
        else
            hipLaunchKernelGGL(calib_accumulate_kernel<NM_BF16>, dim3(tiles), dim3(256), kSlots * kSlotBytes, s, Xc,
                               dc, Tc, (int)K, H);
        const int st = launched();
        if (st != NM_OK)
            return st;
    }
    return NM_OK;
}

int nmk::calib_keep_mask(const void* W, const float* h, int64_t h_stride, int64_t R, int64_t K, int N, int M, int dtype,
                         uint8_t* keep, void* stream)
{
    const int64_t nunits = R * (K / 8);
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
