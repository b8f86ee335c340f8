// gdn_math.hpp -- elementwise helpers on the hardware transcendental units
// (gfx950), internal.
//
// v_exp_f32 (2^x) and v_rcp_f32 / v_rsq_f32 are each accurate to about one
// fp32 ulp.  They are used where the result is rounded to bf16 or enters an
// fp32 output whose tolerance is far above fp32 rounding, in place of the
// correctly rounded library sequences (about 25 instructions per SiLU).
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

// silu(x) = x / (1 + e^{-x}) with e^{-x} = 2^{-x log2(e)}.  Large |x|
// saturate to the right limits: e^{-x} -> inf gives -0, e^{-x} -> 0 gives x.
__device__ __forceinline__ float silu_fast(float x) {
  constexpr float kLog2e = 1.4426950408889634f;
  return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

// 1 / sqrt(x)
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }

}  // namespace gdn
