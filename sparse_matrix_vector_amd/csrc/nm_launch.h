// nm_launch.h -- the kernel side of libnmspmv's entry points.
//
// Each nmk:: call queues (or, where the entry point waits, runs) the work of
// the nm_* entry point of the same name in include/nmspmv.h, on arguments
// that entry point has already checked with nm_rules.h: dtype one of the two,
// shapes within the limits, pointers aligned, outputs disjoint from inputs,
// and at least one row (and K > 0 where the entry point says so).  They
// return NM_OK, NM_ERR_HIP, or the data errors the header lists for the
// entry point (a bad keep-mask, a NaN under the magnitude rule).
//
// Plain C++ declarations, no HIP types: the entry points (nmapi.cpp) are
// host-only code.  The definitions live with the kernels (nmspmv.hip,
// nmcalib.hip).
#ifndef NM_LAUNCH_H
#define NM_LAUNCH_H

#include <cstdint>

namespace nmk {

// y[0 .. n) = +0 (16-bit words); n > 0.
int zero(void* y, int64_t n, void* stream);

// total = sum of R[i] > 0, K > 0; parts with R[i] == 0 are skipped.  workspace:
// NULL, or kSplitWorkspaceBytes (nm_plan.h) of device memory, 256-byte
// aligned, whose counters are zero, for the K-split plan of batched products
// on few rows.
int spmv_multi(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t total,
               int64_t K, int N, int M, int dtype, const void* x, int B, void* const* y, void* workspace,
               void* stream);
int gemv_dense_multi(int count, const void* const* W, const int64_t* R, int64_t total, int64_t K, int dtype,
                     const void* x, int B, void* const* y, void* workspace, void* stream);

// The library's own workspace for allocation-free calls (one per GPU, shared
// by every such call on it): its device address for the current device.
int static_workspace(void** out, void* stream);

// R > 0, K > 0.
int spmv_swiglu(const void* values_gate, const uint8_t* masks_gate, const void* values_up, const uint8_t* masks_up,
                int64_t R, int64_t K, int N, int M, int dtype, const void* x, int B, void* h, void* stream);
int gemv_dense_swiglu(const void* W_gate, const void* W_up, int64_t R, int64_t K, int dtype, const void* x, int B,
                      void* h, void* stream);

// R * K > 0; waits for its work.
int pack(const void* W, const uint8_t* keep, int64_t R, int64_t K, int N, int M, int dtype, void* values,
         uint8_t* masks, void* stream);

// R > 0.
int hybrid_row_loss(const void* W, const uint8_t* keep, const float* h, int64_t h_stride, int64_t R, int64_t K, int N,
                    int M, int dtype, double* loss, void* stream);
int hybrid_select_rows(const double* loss, int64_t R, int64_t n_dense, uint8_t* flags, void* stream);
int hybrid_pack(const void* W, const uint8_t* keep, const uint8_t* flags, int64_t n_dense, int64_t R, int64_t K, int N,
                int M, int dtype, void* values, uint8_t* masks, void* W_dense, int32_t* rows_sparse,
                int32_t* rows_dense, void* stream);

// R > 0, K > 0.
int spmv_hybrid(const void* values, const uint8_t* masks, const int32_t* rows_sparse, const void* W_dense,
                const int32_t* rows_dense, int64_t n_dense, int64_t R, int64_t K, int N, int M, int dtype,
                const void* x, int B, void* y, void* stream);

// T > 0, K > 0.
int calib_accumulate(const void* X, const uint8_t* decode, int64_t T, int64_t K, int dtype, float* H, void* stream);
// R * K > 0.
int calib_keep_mask(const void* W, const float* h, int64_t h_stride, int64_t R, int64_t K, int N, int M, int dtype,
                    uint8_t* keep, void* stream);

}  // namespace nmk

#endif  // NM_LAUNCH_H
