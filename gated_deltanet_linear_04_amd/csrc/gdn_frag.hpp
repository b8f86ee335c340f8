// gdn_frag.hpp -- MFMA operand fragments for gfx950 (wave64), internal.
//
// Every matrix product in this library is built from 16x16 output tiles and
// "k-groups" of 32 contraction indices.  For a k-group, lane l of the wave
// (row/column index l % 16, lane group g = l / 16) holds 8 operand values,
// value j standing for contraction index
//
//     perm(g, j) = 4g + j          (j < 4)
//                  16 + 4g + j-4   (j >= 4)
//
// A and B operands always use this same map, so the MFMA's own assignment of
// (lane, register) to k never matters.  The map is chosen so that the fp32
// accumulator of a previous product -- whose 16x16 C tile gives lane group g
// the rows 4g..4g+3 -- turns into the B operand of the next product without
// any data movement: two stacked C tiles (rows 0..15 and 16..31 of the
// k-group) are exactly the 8 values of perm(g, 0..7).
//
// bf16 operands use one v_mfma_f32_16x16x32_bf16 per k-group; fp32 operands
// use eight v_mfma_f32_16x16x4_f32 (one per j), which keeps fp32 inputs exact
// in the products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Frag;

template <>
struct Frag<__bf16> {
  bf16x8 v;
};

template <>
struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ void mma(f32x4& acc, const Frag<__bf16>& a,
                                    const Frag<__bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a,
                                    const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// Operand values of one lane from a row whose contraction index is
// contiguous: p points at element 0 of the k-group within that row.
__device__ __forceinline__ Frag<__bf16> load_frag(const __bf16* p, int g) {
  const uint2 lo = *reinterpret_cast<const uint2*>(p + 4 * g);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 16 + 4 * g);
  uint4 u;
  u.x = lo.x;
  u.y = lo.y;
  u.z = hi.x;
  u.w = hi.y;
  Frag<__bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u);
  return f;
}

__device__ __forceinline__ Frag<float> load_frag(const float* p, int g) {
  const float4 lo = *reinterpret_cast<const float4*>(p + 4 * g);
  const float4 hi = *reinterpret_cast<const float4*>(p + 16 + 4 * g);
  Frag<float> f;
  f.v[0] = lo.x;
  f.v[1] = lo.y;
  f.v[2] = lo.z;
  f.v[3] = lo.w;
  f.v[4] = hi.x;
  f.v[5] = hi.y;
  f.v[6] = hi.z;
  f.v[7] = hi.w;
  return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> zero_frag();

template <>
__device__ __forceinline__ Frag<__bf16> zero_frag<__bf16>() {
  Frag<__bf16> f;
  f.v = __builtin_bit_cast(bf16x8, uint4{0u, 0u, 0u, 0u});
  return f;
}

template <>
__device__ __forceinline__ Frag<float> zero_frag<float>() {
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
  return f;
}

// Pre-packed fragment: 8 consecutive values per lane (16 B bf16, 32 B fp32).
__device__ __forceinline__ Frag<__bf16> load_packed(const __bf16* p) {
  Frag<__bf16> f;
  f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  return f;
}

__device__ __forceinline__ Frag<float> load_packed(const float* p) {
  const float4 lo = reinterpret_cast<const float4*>(p)[0];
  const float4 hi = reinterpret_cast<const float4*>(p)[1];
  Frag<float> f;
  f.v[0] = lo.x;
  f.v[1] = lo.y;
  f.v[2] = lo.z;
  f.v[3] = lo.w;
  f.v[4] = hi.x;
  f.v[5] = hi.y;
  f.v[6] = hi.z;
  f.v[7] = hi.w;
  return f;
}

__device__ __forceinline__ void store_packed(__bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (__bf16)x[j];
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}

__device__ __forceinline__ void store_packed(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = float4{x[0], x[1], x[2], x[3]};
  reinterpret_cast<float4*>(p)[1] = float4{x[4], x[5], x[6], x[7]};
}

// B operand of a k-group from two stacked accumulator tiles (rows 0..15 and
// 16..31 of the k-group), each row r scaled by s0[r] / s1[r] before rounding.
__device__ __forceinline__ Frag<__bf16> frag_from_acc(const f32x4& c0,
                                                      const f32x4& c1) {
  Frag<__bf16> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = (__bf16)c0[j];
    f.v[4 + j] = (__bf16)c1[j];
  }
  return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_from_acc_t(const f32x4& c0,
                                                   const f32x4& c1);

template <>
__device__ __forceinline__ Frag<__bf16> frag_from_acc_t<__bf16>(
    const f32x4& c0, const f32x4& c1) {
  return frag_from_acc(c0, c1);
}

template <>
__device__ __forceinline__ Frag<float> frag_from_acc_t<float>(const f32x4& c0,
                                                              const f32x4& c1) {
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = c0[j];
    f.v[4 + j] = c1[j];
  }
  return f;
}

// Contraction index of value j in lane group g (see the map above).
__device__ __forceinline__ int kperm(int g, int j) {
  return (j < 4) ? (4 * g + j) : (16 + 4 * g + (j - 4));
}

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) {
  return (__bf16)x;
}
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}

}  // namespace gdn
