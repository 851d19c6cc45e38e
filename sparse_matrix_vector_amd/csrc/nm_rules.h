// nm_rules.h -- libnmspmv's argument rules: the shape limits and pointer
// checks that every entry point applies before it queues any work.
//
// Host-only C++ (no HIP headers): the entry points in nmapi.cpp use it, and
// so can a plain C++ compiler, with sanitizers, for testing the checks
// without a GPU.
#ifndef NM_RULES_H
#define NM_RULES_H

#include <cstddef>
#include <cstdint>

#include "nmspmv.h"

namespace nmh {

constexpr int kMaxBatch = 32;        // activation vectors per call
constexpr int kVectorMaxBatch = 8;   // the VALU kernels' limit; larger batches use the matrix cores
constexpr int kMaxParts = 4;         // matrices one nm_spmv_multi / nm_gemv_dense_multi call takes
constexpr int64_t kCalibMaxK = 65536;   // nm_calib_accumulate: H is K x K fp32 (16 GiB at the limit)

// Row indices are 32-bit in the kernels, and a launch rounds its rows up to
// whole tiles and blocks (at most a few hundred rows past R): R, and a fused
// launch's total, stay below kRowLimit.
constexpr int64_t kRowLimit = (int64_t(1) << 31) - 1024;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Whether [a, a + na) and [b, b + nb) share a byte; an empty or absent buffer
// overlaps nothing.
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (na == 0 || nb == 0 || !a || !b)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// A pointer may be NULL only when its buffer is empty.
inline bool ptr_ok(const void* p, size_t bytes, uintptr_t align)
{
    if (bytes == 0)
        return true;
    return p != nullptr && aligned(p, align);
}

inline int check_dtype(int dtype) { return (dtype == NM_FP16 || dtype == NM_BF16) ? NM_OK : NM_ERR_UNSUPPORTED; }

inline int check_rk(int64_t R, int64_t K)
{
    if (R < 0 || K < 0 || R >= kRowLimit || K > INT32_MAX || K % 8 != 0)
        return NM_ERR_BAD_SHAPE;
    return NM_OK;
}

inline int check_nm(int64_t K, int N, int M)
{
    if ((M != 4 && M != 8) || N < 1 || N >= M || K % M != 0)
        return NM_ERR_BAD_SHAPE;
    return NM_OK;
}

inline int check_batch(int B) { return (B < 1 || B > kMaxBatch) ? NM_ERR_BAD_SHAPE : NM_OK; }

}  // namespace nmh

#endif  // NM_RULES_H
