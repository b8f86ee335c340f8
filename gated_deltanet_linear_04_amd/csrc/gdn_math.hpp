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

// Cross-lane moves through the data-parallel-primitive (DPP) path of the
// vector ALU, instead of LDS-routed permutes.  Controls (gfx9 encoding):
// quad_perm 0x00-0xff, row_shr:n 0x110 + n, row_mirror 0x140,
// row_half_mirror 0x141, row_bcast:15 0x142, row_bcast:31 0x143.  A lane
// whose source lies outside its row, or whose row is masked off, reads 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, ROW_MASK, 0xf, false);
  const int hi =
      __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) |
                                          (unsigned long long)(unsigned)lo));
}

// Sum over the 16 lanes of each row (lanes 16i..16i+15), in every lane of
// the row: pairs, quads, half rows, rows.  Needs the whole wave active.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror: lane i <- 7 - i in its half row
  x += dpp_f32<0x140>(x);  // row_mirror: lane i <- 15 - i in its row
  return x;
}

// Sum over the four lanes of each row that share lane % 4 (4, 8 and 12
// apart), by rotations of the row (row_ror:4, row_ror:8).
__device__ __forceinline__ float row_sum_stride4(float x) {
  x += dpp_f32<0x124>(x);
  x += dpp_f32<0x128>(x);
  return x;
}

// Sum of the lanes 16 apart within each half of the wave (rows 0 and 1, 2
// and 3), in every lane of both rows: one row swap (v_permlane16_swap).
// The same bits as adding the value of the lane 16 apart.
__device__ __forceinline__ float row_pair_sum(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Sum of the lanes 32 apart (the two halves of the wave): one half swap
// (v_permlane32_swap).  The same bits as adding the value of the lane 32
// apart.
__device__ __forceinline__ float half_pair_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order
// (Hillis-Steele within each row, then the row totals carried across rows).
// Needs the whole wave active.
__device__ __forceinline__ double wave_prefix_sum(double x) {
  x += dpp_f64<0x111>(x);       // row_shr:1
  x += dpp_f64<0x112>(x);       // row_shr:2
  x += dpp_f64<0x114>(x);       // row_shr:4
  x += dpp_f64<0x118>(x);       // row_shr:8
  x += dpp_f64<0x142, 0xa>(x);  // row 0's total into row 1, row 2's into row 3
  x += dpp_f64<0x143, 0xc>(x);  // lanes 0..31's total into rows 2 and 3
  return x;
}

}  // namespace gdn
