// nmapi.cpp -- libnmspmv's C entry points (include/nmspmv.h): argument checks,
// then the kernel side (nm_launch.h).
//
// Every call validates its whole argument list here, before any work is
// queued: dtype, shapes and their limits (nm_rules.h), pointer presence and
// alignment, outputs that overlap an input or each other; then it settles the
// empty cases (no rows: nothing to do; K = 0: outputs are zero) and hands the
// rest to the kernels.  Host-only C++: no HIP headers and no device code, so
// a plain C++ compiler can build these checks with sanitizers for testing.
#include <cstddef>
#include <cstdint>

#include "nm_launch.h"
#include "nm_plan.h"
#include "nm_rules.h"
#include "nmspmv.h"

using namespace nmh;

namespace {

int zero_outputs(int count, void* const* y, const int64_t* R, int B, void* stream)
{
    for (int i = 0; i < count; ++i) {
        if (R[i] == 0)
            continue;
        const int st = nmk::zero(y[i], (int64_t)B * R[i], stream);
        if (st != NM_OK)
            return st;
    }
    return NM_OK;
}

}  // namespace

namespace {

// nm_spmv_multi with an optional K-split workspace (ws, ws_bytes; checked
// here when given) or, with use_static, the library's own.
int spmv_multi_with(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t K,
                    int N, int M, int dtype, const void* x, int B, void* const* y, void* ws, int64_t ws_bytes,
                    bool use_static, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if (count < 1 || count > kMaxParts || !R)
        return count < 1 || count > kMaxParts ? NM_ERR_BAD_SHAPE : NM_ERR_INVALID_ARG;
    if ((st = check_rk(0, K)) != NM_OK || (st = check_nm(K, N, M)) != NM_OK || (st = check_batch(B)) != NM_OK)
        return st;
    int64_t total = 0;
    for (int i = 0; i < count; ++i) {
        if ((st = check_rk(R[i], K)) != NM_OK)
            return st;
        total += R[i];
    }
    if (total >= kRowLimit)
        return NM_ERR_BAD_SHAPE;
    if (!values || !masks || !y)
        return NM_ERR_INVALID_ARG;
    const size_t xbytes = (size_t)B * (size_t)K * 2;
    if (!ptr_ok(x, xbytes, 16))
        return NM_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
        const size_t vb = (size_t)R[i] * (size_t)(K / M * N) * 2, mb = (size_t)R[i] * (size_t)(K / 8);
        const size_t yb = (size_t)B * (size_t)R[i] * 2;
        if (!ptr_ok(values[i], vb, 16) || !ptr_ok(masks[i], mb, 16) || !ptr_ok(y[i], yb, 2))
            return NM_ERR_INVALID_ARG;
        if (overlaps(y[i], yb, x, xbytes))
            return NM_ERR_INVALID_ARG;
        for (int j = 0; j < count; ++j) {
            const size_t vbj = (size_t)R[j] * (size_t)(K / M * N) * 2, mbj = (size_t)R[j] * (size_t)(K / 8);
            if (overlaps(y[i], yb, values[j], vbj) || overlaps(y[i], yb, masks[j], mbj) ||
                (j != i && overlaps(y[i], yb, y[j], (size_t)B * (size_t)R[j] * 2)))
                return NM_ERR_INVALID_ARG;
        }
    }
    if (ws) {
        if (ws_bytes < (int64_t)kSplitWorkspaceBytes || !aligned(ws, 256))
            return NM_ERR_INVALID_ARG;
        if (overlaps(ws, (size_t)ws_bytes, x, xbytes))
            return NM_ERR_INVALID_ARG;
        for (int i = 0; i < count; ++i) {
            const size_t vb = (size_t)R[i] * (size_t)(K / M * N) * 2, mb = (size_t)R[i] * (size_t)(K / 8);
            if (overlaps(ws, (size_t)ws_bytes, values[i], vb) || overlaps(ws, (size_t)ws_bytes, masks[i], mb) ||
                overlaps(ws, (size_t)ws_bytes, y[i], (size_t)B * (size_t)R[i] * 2))
                return NM_ERR_INVALID_ARG;
        }
    }
    if (total == 0)
        return NM_OK;
    if (K == 0)
        return zero_outputs(count, y, R, B, stream);
    if (use_static && (st = nmk::static_workspace(&ws, stream)) != NM_OK)
        return st;
    return nmk::spmv_multi(count, values, masks, R, total, K, N, M, dtype, x, B, y, ws, stream);
}

int gemv_dense_multi_with(int count, const void* const* W, const int64_t* R, int64_t K, int dtype, const void* x,
                          int B, void* const* y, void* ws, int64_t ws_bytes, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if (count < 1 || count > kMaxParts || !R)
        return count < 1 || count > kMaxParts ? NM_ERR_BAD_SHAPE : NM_ERR_INVALID_ARG;
    if ((st = check_rk(0, K)) != NM_OK || (st = check_batch(B)) != NM_OK)
        return st;
    int64_t total = 0;
    for (int i = 0; i < count; ++i) {
        if ((st = check_rk(R[i], K)) != NM_OK)
            return st;
        total += R[i];
    }
    if (total >= kRowLimit)
        return NM_ERR_BAD_SHAPE;
    if (!W || !y)
        return NM_ERR_INVALID_ARG;
    const size_t xbytes = (size_t)B * (size_t)K * 2;
    if (!ptr_ok(x, xbytes, 16))
        return NM_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
        const size_t wb = (size_t)R[i] * (size_t)K * 2, yb = (size_t)B * (size_t)R[i] * 2;
        if (!ptr_ok(W[i], wb, 16) || !ptr_ok(y[i], yb, 2))
            return NM_ERR_INVALID_ARG;
        if (overlaps(y[i], yb, x, xbytes))
            return NM_ERR_INVALID_ARG;
        for (int j = 0; j < count; ++j)
            if (overlaps(y[i], yb, W[j], (size_t)R[j] * (size_t)K * 2) ||
                (j != i && overlaps(y[i], yb, y[j], (size_t)B * (size_t)R[j] * 2)))
                return NM_ERR_INVALID_ARG;
    }
    if (ws) {
        if (ws_bytes < (int64_t)kSplitWorkspaceBytes || !aligned(ws, 256))
            return NM_ERR_INVALID_ARG;
        if (overlaps(ws, (size_t)ws_bytes, x, xbytes))
            return NM_ERR_INVALID_ARG;
        for (int i = 0; i < count; ++i)
            if (overlaps(ws, (size_t)ws_bytes, W[i], (size_t)R[i] * (size_t)K * 2) ||
                overlaps(ws, (size_t)ws_bytes, y[i], (size_t)B * (size_t)R[i] * 2))
                return NM_ERR_INVALID_ARG;
    }
    if (total == 0)
        return NM_OK;
    if (K == 0)
        return zero_outputs(count, y, R, B, stream);
    return nmk::gemv_dense_multi(count, W, R, total, K, dtype, x, B, y, ws, stream);
}

}  // namespace

extern "C" {

int nm_version(void) { return 101; }

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

int nm_spmv_multi(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t K,
                  int N, int M, int dtype, const void* x, int B, void* const* y, void* stream)
{
    return spmv_multi_with(count, values, masks, R, K, N, M, dtype, x, B, y, nullptr, 0, false, stream);
}

int nm_spmv_multi_ws(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t K,
                     int N, int M, int dtype, const void* x, int B, void* const* y, void* workspace,
                     int64_t workspace_bytes, void* stream)
{
    return spmv_multi_with(count, values, masks, R, K, N, M, dtype, x, B, y, workspace, workspace_bytes, false,
                           stream);
}

int nm_spmv_multi_noalloc(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R,
                          int64_t K, int N, int M, int dtype, const void* x, int B, void* const* y, void* stream)
{
    return spmv_multi_with(count, values, masks, R, K, N, M, dtype, x, B, y, nullptr, 0, true, stream);
}

int64_t nm_workspace_bytes(void) { return (int64_t)kSplitWorkspaceBytes; }

int nm_spmv(const void* values, const uint8_t* masks, int64_t R, int64_t K, int N, int M, int dtype, const void* x,
            int B, void* y, void* stream)
{
    return nm_spmv_multi(1, &values, &masks, &R, K, N, M, dtype, x, B, &y, stream);
}

int nm_gemv_dense_multi(int count, const void* const* W, const int64_t* R, int64_t K, int dtype, const void* x, int B,
                        void* const* y, void* stream)
{
    return gemv_dense_multi_with(count, W, R, K, dtype, x, B, y, nullptr, 0, stream);
}

int nm_gemv_dense_multi_ws(int count, const void* const* W, const int64_t* R, int64_t K, int dtype, const void* x,
                           int B, void* const* y, void* workspace, int64_t workspace_bytes, void* stream)
{
    return gemv_dense_multi_with(count, W, R, K, dtype, x, B, y, workspace, workspace_bytes, stream);
}

int nm_gemv_dense(const void* W, int64_t R, int64_t K, int dtype, const void* x, int B, void* y, void* stream)
{
    return nm_gemv_dense_multi(1, &W, &R, K, dtype, x, B, &y, stream);
}

int nm_spmv_swiglu(const void* values_gate, const uint8_t* masks_gate, const void* values_up, const uint8_t* masks_up,
                   int64_t R, int64_t K, int N, int M, int dtype, const void* x, int B, void* h, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK || (st = check_nm(K, N, M)) != NM_OK || (st = check_batch(B)) != NM_OK)
        return st;
    if (2 * R >= kRowLimit)                      // the launch interleaves the gate and up rows
        return NM_ERR_BAD_SHAPE;
    const size_t xbytes = (size_t)B * (size_t)K * 2, hbytes = (size_t)B * (size_t)R * 2;
    const size_t vb = (size_t)R * (size_t)(K / M * N) * 2, mb = (size_t)R * (size_t)(K / 8);
    if (!ptr_ok(x, xbytes, 16) || !ptr_ok(h, hbytes, 2) || !ptr_ok(values_gate, vb, 16) ||
        !ptr_ok(masks_gate, mb, 16) || !ptr_ok(values_up, vb, 16) || !ptr_ok(masks_up, mb, 16))
        return NM_ERR_INVALID_ARG;
    if (overlaps(h, hbytes, x, xbytes) || overlaps(h, hbytes, values_gate, vb) || overlaps(h, hbytes, masks_gate, mb) ||
        overlaps(h, hbytes, values_up, vb) || overlaps(h, hbytes, masks_up, mb))
        return NM_ERR_INVALID_ARG;
    if (R == 0)
        return NM_OK;
    if (K == 0)                                  // SiLU(0) * 0
        return nmk::zero(h, (int64_t)B * R, stream);
    return nmk::spmv_swiglu(values_gate, masks_gate, values_up, masks_up, R, K, N, M, dtype, x, B, h, stream);
}

int nm_gemv_dense_swiglu(const void* W_gate, const void* W_up, int64_t R, int64_t K, int dtype, const void* x, int B,
                         void* h, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK || (st = check_batch(B)) != NM_OK)
        return st;
    if (2 * R >= kRowLimit)
        return NM_ERR_BAD_SHAPE;
    const size_t xbytes = (size_t)B * (size_t)K * 2, hbytes = (size_t)B * (size_t)R * 2;
    const size_t wb = (size_t)R * (size_t)K * 2;
    if (!ptr_ok(x, xbytes, 16) || !ptr_ok(h, hbytes, 2) || !ptr_ok(W_gate, wb, 16) || !ptr_ok(W_up, wb, 16))
        return NM_ERR_INVALID_ARG;
    if (overlaps(h, hbytes, x, xbytes) || overlaps(h, hbytes, W_gate, wb) || overlaps(h, hbytes, W_up, wb))
        return NM_ERR_INVALID_ARG;
    if (R == 0)
        return NM_OK;
    if (K == 0)
        return nmk::zero(h, (int64_t)B * R, stream);
    return nmk::gemv_dense_swiglu(W_gate, W_up, R, K, dtype, x, B, h, stream);
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
    if (R == 0 || K == 0)
        return NM_OK;
    return nmk::pack(W, keep, R, K, N, M, dtype, values, masks, stream);
}

int nm_hybrid_row_loss(const void* W, const uint8_t* keep, const float* h, int64_t h_stride, int64_t R, int64_t K, int N,
                       int M, int dtype, double* loss, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK || (st = check_nm(K, N, M)) != NM_OK)
        return st;
    if (h && h_stride < 1)
        return NM_ERR_BAD_SHAPE;
    const size_t wbytes = (size_t)R * (size_t)K * 2, kbytes = keep ? (size_t)R * (size_t)K : 0;
    const size_t hbytes = h && K > 0 ? ((size_t)(K - 1) * (size_t)h_stride + 1) * 4 : 0;
    const size_t lbytes = (size_t)R * 8;
    if (!ptr_ok(W, wbytes, 2) || !ptr_ok(loss, lbytes, 8) || (h && !ptr_ok(h, hbytes, 4)))
        return NM_ERR_INVALID_ARG;
    if (overlaps(loss, lbytes, W, wbytes) || overlaps(loss, lbytes, keep, kbytes) || overlaps(loss, lbytes, h, hbytes))
        return NM_ERR_INVALID_ARG;
    if (R == 0)
        return NM_OK;
    return nmk::hybrid_row_loss(W, keep, h, h_stride, R, K, N, M, dtype, loss, stream);
}

int nm_hybrid_select_rows(const double* loss, int64_t R, int64_t n_dense, uint8_t* flags, void* stream)
{
    if (R < 0 || R >= kRowLimit || n_dense < 0 || n_dense > R)
        return NM_ERR_BAD_SHAPE;
    if (!ptr_ok(loss, (size_t)R * 8, 8) || !ptr_ok(flags, (size_t)R, 1) || overlaps(flags, (size_t)R, loss, (size_t)R * 8))
        return NM_ERR_INVALID_ARG;
    if (R == 0)
        return NM_OK;
    return nmk::hybrid_select_rows(loss, R, n_dense, flags, stream);
}

int nm_hybrid_pack(const void* W, const uint8_t* keep, const uint8_t* flags, int64_t n_dense, int64_t R, int64_t K,
                   int N, int M, int dtype, void* values, uint8_t* masks, void* W_dense, int32_t* rows_sparse,
                   int32_t* rows_dense, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK || (st = check_nm(K, N, M)) != NM_OK)
        return st;
    if (n_dense < 0 || n_dense > R)
        return NM_ERR_BAD_SHAPE;
    const int64_t Rs = R - n_dense;
    const size_t wbytes = (size_t)R * (size_t)K * 2, kbytes = keep ? (size_t)R * (size_t)K : 0;
    const size_t vbytes = (size_t)Rs * (size_t)(K / M * N) * 2, mbytes = (size_t)Rs * (size_t)(K / 8);
    const size_t dbytes = (size_t)n_dense * (size_t)K * 2;
    const size_t sbytes = (size_t)Rs * 4, ibytes = (size_t)n_dense * 4;
    if (!ptr_ok(W, wbytes, 16) || !ptr_ok(flags, (size_t)R, 1) || !ptr_ok(values, vbytes, 16) ||
        !ptr_ok(masks, mbytes, 16) || !ptr_ok(W_dense, dbytes, 16) || !ptr_ok(rows_sparse, sbytes, 4) ||
        !ptr_ok(rows_dense, ibytes, 4))
        return NM_ERR_INVALID_ARG;
    const void* outs[5] = {values, masks, W_dense, rows_sparse, rows_dense};
    const size_t osz[5] = {vbytes, mbytes, dbytes, sbytes, ibytes};
    for (int i = 0; i < 5; ++i) {
        if (overlaps(outs[i], osz[i], W, wbytes) || overlaps(outs[i], osz[i], keep, kbytes) ||
            overlaps(outs[i], osz[i], flags, (size_t)R))
            return NM_ERR_INVALID_ARG;
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], osz[i], outs[j], osz[j]))
                return NM_ERR_INVALID_ARG;
    }
    if (R == 0)
        return NM_OK;
    return nmk::hybrid_pack(W, keep, flags, n_dense, R, K, N, M, dtype, values, masks, W_dense, rows_sparse, rows_dense,
                            stream);
}

int nm_spmv_hybrid(const void* values, const uint8_t* masks, const int32_t* rows_sparse, const void* W_dense,
                   const int32_t* rows_dense, int64_t n_dense, int64_t R, int64_t K, int N, int M, int dtype,
                   const void* x, int B, void* y, void* stream)
{
    int st = check_dtype(dtype);
    if (st != NM_OK)
        return st;
    if ((st = check_rk(R, K)) != NM_OK || (st = check_nm(K, N, M)) != NM_OK || (st = check_batch(B)) != NM_OK)
        return st;
    if (n_dense < 0 || n_dense > R)
        return NM_ERR_BAD_SHAPE;
    const int64_t Rs = R - n_dense;
    const size_t vbytes = (size_t)Rs * (size_t)(K / M * N) * 2, mbytes = (size_t)Rs * (size_t)(K / 8);
    const size_t dbytes = (size_t)n_dense * (size_t)K * 2, sbytes = (size_t)Rs * 4, ibytes = (size_t)n_dense * 4;
    const size_t xbytes = (size_t)B * (size_t)K * 2, ybytes = (size_t)B * (size_t)R * 2;
    if (!ptr_ok(values, vbytes, 16) || !ptr_ok(masks, mbytes, 16) || !ptr_ok(rows_sparse, sbytes, 4) ||
        !ptr_ok(W_dense, dbytes, 16) || !ptr_ok(rows_dense, ibytes, 4) || !ptr_ok(x, xbytes, 16) ||
        !ptr_ok(y, ybytes, 2))
        return NM_ERR_INVALID_ARG;
    if (overlaps(y, ybytes, values, vbytes) || overlaps(y, ybytes, masks, mbytes) || overlaps(y, ybytes, W_dense, dbytes) ||
        overlaps(y, ybytes, rows_sparse, sbytes) || overlaps(y, ybytes, rows_dense, ibytes) ||
        overlaps(y, ybytes, x, xbytes))
        return NM_ERR_INVALID_ARG;
    if (R == 0)
        return NM_OK;
    if (K == 0)
        return nmk::zero(y, (int64_t)B * R, stream);
    return nmk::spmv_hybrid(values, masks, rows_sparse, W_dense, rows_dense, n_dense, R, K, N, M, dtype, x, B, y,
                            stream);
}

int nm_calib_accumulate(const void* X, const uint8_t* decode, int64_t T, int64_t K, int dtype, float* H, void* stream)
{
    if (check_dtype(dtype) != NM_OK)
        return NM_ERR_UNSUPPORTED;
    if (T < 0 || K < 0 || K % 8 != 0 || T > INT32_MAX || K > kCalibMaxK)
        return NM_ERR_BAD_SHAPE;
    const size_t xbytes = (size_t)T * (size_t)K * 2, hbytes = (size_t)K * (size_t)K * 4;
    if (!ptr_ok(X, xbytes, 16) || !ptr_ok(H, hbytes, 4))
        return NM_ERR_INVALID_ARG;
    if (overlaps(H, hbytes, X, xbytes) || overlaps(H, hbytes, decode, (size_t)T))
        return NM_ERR_INVALID_ARG;
    if (T == 0 || K == 0)
        return NM_OK;
    return nmk::calib_accumulate(X, decode, T, K, dtype, H, stream);
}

int nm_calib_keep_mask(const void* W, const float* h, int64_t h_stride, int64_t R, int64_t K, int N, int M, int dtype,
                       uint8_t* keep, void* stream)
{
    if (check_dtype(dtype) != NM_OK)
        return NM_ERR_UNSUPPORTED;
    if (check_rk(R, K) != NM_OK || check_nm(K, N, M) != NM_OK || h_stride < 1)   // the shape rules of nm_pack
        return NM_ERR_BAD_SHAPE;
    const size_t wbytes = (size_t)R * (size_t)K * 2, kbytes = (size_t)R * (size_t)K;
    const size_t hbytes = K > 0 ? ((size_t)(K - 1) * (size_t)h_stride + 1) * 4 : 0;
    if (!ptr_ok(W, wbytes, 16) || !ptr_ok(keep, kbytes, 8) || !ptr_ok(h, hbytes, 4))
        return NM_ERR_INVALID_ARG;
    if (overlaps(keep, kbytes, W, wbytes) || overlaps(keep, kbytes, h, hbytes))
        return NM_ERR_INVALID_ARG;
    if (R == 0 || K == 0)
        return NM_OK;
    return nmk::calib_keep_mask(W, h, h_stride, R, K, N, M, dtype, keep, stream);
}

}  // extern "C"
