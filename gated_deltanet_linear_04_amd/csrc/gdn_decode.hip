// gdn_decode.hip -- one recurrent step of the gated delta rule per request,
// on a state cache addressed by slot (gfx950).
//
// A request is one new token of a sequence whose state S (Dv x Dk fp32,
// row-major, the same layout as the prefill's state) sits in
// cache[slot][h].  Per value head h (key head h / r), with the gate, beta,
// L2 norm and gated RMSNorm of "Add opt-in fused Qwen3.5 inference kernels"
// (JevAny PR #29), Summary, and the recurrent form those kernels evaluate in
// chunks:
//   g  = -exp(A_log[h]) softplus(a + dt_bias[h]),   beta = sigmoid(b)
//   k^ = k / sqrt(|k|^2 + eps),   q^ = scale q / sqrt(|q|^2 + eps)
//   S  = e^g S;   S = S + beta (v - S k^) k^T;   o = S q^
//   y  = o / sqrt(mean(o^2) + eps_n) * w * silu(z)     (when z, w are given)
// The step reads and writes the 64 KB state once and touches ~1 KB of
// token data, so it is HBM-bound on the state: every product is a
// matrix-vector product done in fp32 on the vector ALUs (no MFMA shape).
//
// Block = (request, value head), 256 threads.  Thread t = 4 r0 + j owns
// state rows r0 and r0 + 64, columns 16 u + 4 j .. 16 u + 4 j + 3 for
// u = 0..7: a wave's 16-byte loads cover 16 rows x 64 contiguous bytes per
// instruction, and the four threads of a row (one DPP quad) reduce a row's
// dot products in two DPP steps.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_decode.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

template <typename T>
struct DecodeArgs {
  const T *q, *k, *v, *a, *b, *z;
  const float *A_log, *dt_bias, *norm_w;
  float* cache;
  const int32_t* slots;
  int64_t num_slots;
  int Hk, Hv, r;
  float scale, l2_eps, norm_eps;
  T* o;
};

// Four consecutive q or k elements, kept in their stored form until used
// (bf16 stays packed: half the registers of fp32).
template <typename T>
struct Vec4;

template <>
struct Vec4<float> {
  float4 x;
  __device__ __forceinline__ void load(const float* p) {
    x = *reinterpret_cast<const float4*>(p);
  }
  __device__ __forceinline__ float4 get() const { return x; }
};

template <>
struct Vec4<__bf16> {
  uint2 x;
  __device__ __forceinline__ void load(const __bf16* p) {
    x = *reinterpret_cast<const uint2*>(p);
  }
  // bf16 -> fp32 is the 16 bits moved to the top half
  __device__ __forceinline__ float4 get() const {
    return float4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                  __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
  }
};

// Sum over the four lanes of a DPP quad (lanes 4m .. 4m + 3).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, false));
  return x;
}

__device__ __forceinline__ float dot4(const float4& x, const float4& y) {
  return x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
}

// bf16: at most 128 VGPRs, so four blocks fit on a CU
template <typename T>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 4 : 3) void decode_kernel(DecodeArgs<T> p) {
  __shared__ float red[4];
  const int i = blockIdx.x / p.Hv;
  const int h = blockIdx.x - i * p.Hv;
  const int kh = h / p.r;
  const int tid = threadIdx.x, j = tid & 3, r0 = tid >> 2;
  int64_t slot = p.slots ? (int64_t)p.slots[i] : (int64_t)i;
  const bool live = slot >= 0 && slot < p.num_slots;
  if (!live) slot = 0;  // loads stay in bounds; the cache is not written
  float* S = p.cache + (slot * p.Hv + h) * (int64_t)(kHeadDim * kHeadDim);
  float* S0 = S + r0 * kHeadDim + 4 * j;
  float* S1 = S0 + 64 * kHeadDim;

  float4 s0[8], s1[8];
  Vec4<T> kk[8], qq[8];
  const int64_t kq_row = ((int64_t)i * p.Hk + kh) * kHeadDim + 4 * j;
  const int64_t vh = (int64_t)i * p.Hv + h;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    kk[u].load(p.k + kq_row + 16 * u);
    qq[u].load(p.q + kq_row + 16 * u);
  }
  const float v0 = (float)p.v[vh * kHeadDim + r0];
  const float v1 = (float)p.v[vh * kHeadDim + r0 + 64];
  const float av = (float)p.a[vh] + p.dt_bias[h];
  const float bv = (float)p.b[vh];
  const float Al = p.A_log[h];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    s0[u] = *reinterpret_cast<const float4*>(S0 + 16 * u);
    s1[u] = *reinterpret_cast<const float4*>(S1 + 16 * u);
  }
  // every load above is issued before any arithmetic waits for one: the
  // token and state loads share one memory round trip, and the small token
  // loads come first, so (loads complete in order) the token-only dots can
  // start while the state is still arriving
  __builtin_amdgcn_sched_barrier(0);

  // One pass over the old state gives everything the step needs: with
  // S' = e^g S + c k^T (c = beta (v - e^g S k^) rk), S' q = e^g (S q) +
  // c (k . q), so q is consumed before the update.  Dots over the row's 128
  // columns: the four lanes of the quad.
  float ssk = 0.f, ssq = 0.f, kq = 0.f, d0 = 0.f, d1 = 0.f, e0 = 0.f, e1 = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float4 kv = kk[u].get(), qv = qq[u].get();
    ssk += dot4(kv, kv);
    ssq += dot4(qv, qv);
    kq += dot4(kv, qv);
    d0 += dot4(s0[u], kv);
    d1 += dot4(s1[u], kv);
    e0 += dot4(s0[u], qv);
    e1 += dot4(s1[u], qv);
  }
  ssk = quad_sum(ssk);
  ssq = quad_sum(ssq);
  kq = quad_sum(kq);
  d0 = quad_sum(d0);
  d1 = quad_sum(d1);
  e0 = quad_sum(e0);
  e1 = quad_sum(e1);
  const float rk = 1.f / sqrtf(ssk + p.l2_eps);
  const float rq = p.scale / sqrtf(ssq + p.l2_eps);

  // gate and write strength
  const float sp = fmaxf(av, 0.f) + log1pf(expf(-fabsf(av)));
  const float alpha = expf(-expf(Al) * sp);
  const float beta = 1.f / (1.f + expf(-bv));

  // S <- e^g S + c k^T with c = beta (v - e^g S k^) rk, k^ = rk k
  const float c0 = beta * (v0 - alpha * rk * d0) * rk;
  const float c1 = beta * (v1 - alpha * rk * d1) * rk;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float4 kv = kk[u].get();
    s0[u].x = alpha * s0[u].x + c0 * kv.x;
    s0[u].y = alpha * s0[u].y + c0 * kv.y;
    s0[u].z = alpha * s0[u].z + c0 * kv.z;
    s0[u].w = alpha * s0[u].w + c0 * kv.w;
    s1[u].x = alpha * s1[u].x + c1 * kv.x;
    s1[u].y = alpha * s1[u].y + c1 * kv.y;
    s1[u].z = alpha * s1[u].z + c1 * kv.z;
    s1[u].w = alpha * s1[u].w + c1 * kv.w;
  }
  if (live) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      *reinterpret_cast<float4*>(S0 + 16 * u) = s0[u];
      *reinterpret_cast<float4*>(S1 + 16 * u) = s1[u];
    }
  }
  // o = S' q^ for the two rows; padding requests produce zeros
  e0 = (alpha * e0 + c0 * kq) * rq;
  e1 = (alpha * e1 + c1 * kq) * rq;
  if (!live) e0 = e1 = 0.f;

  // lane j = 0 writes row r0, lane j = 1 row r0 + 64
  const int row = r0 + ((j & 1) ? 64 : 0);
  float y = (j & 1) ? e1 : e0;
  if (p.z) {
    // mean of o^2 over the 128 rows: the quads of a wave, then the waves
    float sq = e0 * e0 + e1 * e1;
    sq += __shfl_xor(sq, 4);
    sq += __shfl_xor(sq, 8);
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    if ((tid & 63) == 0) red[tid >> 6] = sq;
    __syncthreads();
    const float ms = (red[0] + red[1] + red[2] + red[3]) * (1.f / kHeadDim);
    const float rinv = 1.f / sqrtf(ms + p.norm_eps);
    const float zf = (float)p.z[vh * kHeadDim + row];
    y = y * rinv * p.norm_w[row] * (zf / (1.f + expf(-zf)));
  }
  if (j < 2) p.o[vh * kHeadDim + row] = (T)y;
}

template <typename T>
hipError_t launch_decode_t(const DecodeLaunch& L, hipStream_t st) {
  DecodeArgs<T> a;
  a.q = static_cast<const T*>(L.q);
  a.k = static_cast<const T*>(L.k);
  a.v = static_cast<const T*>(L.v);
  a.a = static_cast<const T*>(L.a);
  a.b = static_cast<const T*>(L.b);
  a.z = static_cast<const T*>(L.z);
  a.A_log = L.A_log;
  a.dt_bias = L.dt_bias;
  a.norm_w = L.norm_w;
  a.cache = L.cache;
  a.slots = L.slots;
  a.num_slots = L.num_slots;
  a.Hk = L.Hk;
  a.Hv = L.Hv;
  a.r = L.Hv / L.Hk;
  a.scale = L.scale;
  a.l2_eps = L.l2_eps;
  a.norm_eps = L.norm_eps;
  a.o = static_cast<T*>(L.o);
  const unsigned blocks = (unsigned)((int64_t)L.B * L.Hv);
  hipLaunchKernelGGL(decode_kernel<T>, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t st) {
  if (L.B == 0) return hipSuccess;
  return L.dtype == 1 ? launch_decode_t<__bf16>(L, st) : launch_decode_t<float>(L, st);
}

}  // namespace gdn
