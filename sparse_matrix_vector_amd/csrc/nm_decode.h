// nm_decode.h -- exact decoding of 16-bit and fp32 words into double from
// their fields (sign, exponent, fraction), independent of the GPU's denormal
// mode.  Shared by the calibration and hybrid-row kernels, whose decisions
// (keep-masks, dense rows) must not depend on how denormals are handled.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nmspmv.h"

namespace nm_decode {

__device__ __forceinline__ double fields_to_f64(uint32_t bits, int fbits, int ebits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t emax = (1u << ebits) - 1;
    const uint32_t sign = bits >> (fbits + ebits), e = (bits >> fbits) & emax, f = bits & ((1u << fbits) - 1);
    double v;
    if (e == emax)
        v = f ? __builtin_nan("") : __builtin_inf();
    else if (e == 0)
        v = ldexp((double)f, 1 - bias - fbits);
    else
        v = ldexp((double)(f | (1u << fbits)), (int)e - bias - fbits);
    return sign ? -v : v;
}

// A weight word of dtype DT (NM_FP16 or NM_BF16).
template <int DT>
__device__ __forceinline__ double w_to_f64(uint32_t bits)
{
    return DT == NM_FP16 ? fields_to_f64(bits, 10, 5) : fields_to_f64(bits, 7, 8);
}

// An fp32 value, exactly.
__device__ __forceinline__ double f32_to_f64(float v)
{
    return fields_to_f64(__builtin_bit_cast(uint32_t, v), 23, 8);
}

}  // namespace nm_decode
