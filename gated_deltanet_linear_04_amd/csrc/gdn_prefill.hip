// gdn_prefill.hip -- gfx950 kernels of the chunked gated delta rule prefill.
//
// Operator: the gated delta rule of "Add opt-in fused Qwen3.5 inference
// kernels" (JevAny PR #29), Summary -- decay gate from A_log and dt_bias,
// sigmoid beta, q/k L2 norm, grouped value heads, gated RMSNorm after -- at
// the geometry of "feat(qwen35): add SM120 FlashInfer GDN prefill candidate"
// (pegainfer PR #862), Correctness (Hq/Hk/Hv/D = 16/16/32/128, a 128x128
// state per value head).  Neither page prints the algorithm; the chunked
// form below is derived from the recurrence.
//
// Chunked form (C = 64 tokens, H = S^T the dk x dv state at chunk entry,
// gamma the in-chunk cumulative log-decay, rk/rq the inverse L2 norms, rq
// including the q scale, K/Q/V the raw input rows):
//   A_ts  = beta_t e^{gamma_t-gamma_s} rk_t rk_s (K K^T)_ts,  t > s
//   Tb    = (I + A)^{-1} diag(beta)
//   V'    = Tb (V - diag(e^gamma rk) K H)          per-token delta writes
//   O     = diag(e^gamma rq) Q H + MP V',  MP_ts = e^{gamma_t-gamma_s}
//           rq_t rk_s (Q K^T)_ts for s <= t
//   H    <- e^{gamma_L} H + K^T diag(e^{gamma_L-gamma} rk) V'
// Only exponentials of non-positive arguments appear.  The raw bf16 K, Q and
// V enter the MFMAs exactly; every normalisation and gate is a per-row fp32
// factor.
//
// Kernels, in launch order on the caller's stream:
//   prep  : per (chunk, value head): norms, gates, the two Gram products,
//           Tb and MP as packed MFMA fragments (parallel over chunks)
//   chain : per (sequence, value head, 16-column block of the state): the
//           sequential pass over chunks (four waves splitting each chunk's
//           products by rows, state in registers, operands staged by a
//           fifth wave); exports the state at each chunk entry and the
//           delta writes V' as MFMA fragments
//   out   : per (chunk, value head): O = diag(e^gamma rq) Q H + MP V' for
//           all 128 columns, with the gated RMSNorm fused (parallel over
//           chunks)
//
// Chunks never straddle sequences.  Chunk j of sequence n owns workspace
// slot floor(cu[n] / 64) + n + j: slots of different sequences never
// collide and all lie below floor(T / 64) + N, so no prefix sum over the
// sequences (and no extra launch) is needed to place them.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "gdn_frag.hpp"
#include "gdn_internal.hpp"
#include "gdn_math.hpp"

namespace gdn {

// ------------------------------------------------------------ sequences ----

// Token range [s, e) of sequence n, clamped into [0, T] (a malformed
// cu_seqlens then gives unspecified results but every access stays inside
// the tensors and the workspace).
__device__ __forceinline__ void seq_range(const int32_t* cu, int64_t T, int n,
                                          int64_t& s, int64_t& e) {
  if (!cu) {
    s = 0;
    e = T;
    return;
  }
  s = cu[n];
  e = cu[n + 1];
  s = s < 0 ? 0 : (s > T ? T : s);
  e = e < s ? s : (e > T ? T : e);
}

// First workspace slot of sequence n.
__device__ __forceinline__ int64_t slot_base(const int32_t* cu, int64_t T,
                                             int n) {
  int64_t s, e;
  seq_range(cu, T, n, s, e);
  return s / kChunk + n;
}

// Blocks of the prep and output kernels cover (chunk slot, value head) on a
// 1-D grid: unit u = (slot, key head) goes to XCD u % 8 (blocks are dealt
// to XCDs by blockIdx % 8), and its r value heads take consecutive blocks
// there, so the second reader of the unit's q/k rows finds them in that
// XCD's L2.  Returns false for the padding blocks past the last unit.
__device__ __forceinline__ bool slot_head(int bid, int Hk, int r, int64_t slots,
                                          int& c, int& h) {
  const int xcd = bid & 7, k = bid >> 3;
  const int e = k % r;
  const int64_t u = (int64_t)(k / r) * 8 + xcd;
  if (u >= slots * Hk) return false;
  c = (int)(u / Hk);
  h = (int)(u % Hk) * r + e;
  return true;
}

static inline uint64_t slot_head_blocks64(int64_t slots, int Hk, int r) {
  return (uint64_t)((slots * Hk + 7) / 8) * 8 * (uint64_t)r;
}
static inline unsigned slot_head_blocks(int64_t slots, int Hk, int r) {
  return (unsigned)slot_head_blocks64(slots, Hk, r);
}

// Four consecutive values as one 8-byte (bf16) or 16-byte (fp32) store
// (global or LDS).
__device__ __forceinline__ void store4(__bf16* p, const float (&y)[4]) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = (__bf16)y[j];
  *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ void store4(float* p, const float (&y)[4]) {
  *reinterpret_cast<float4*>(p) = float4{y[0], y[1], y[2], y[3]};
}

// Tb and MP are causal 64x64 operands, packed as fragments 2w + kb (row
// tile w, k-group kb of 32 tokens).  Fragments (0, 1) and (1, 1) lie
// wholly above the diagonal: they are neither written nor read.
__device__ __host__ constexpr bool zero_frag_index(int f) { return f == 1 || f == 3; }

// ---------------------------------------------------------------- prep ----

// Element j of a 16-byte piece (j a compile-time index after unrolling).
template <typename T>
__device__ __forceinline__ T elem(const uint4& x, int j);
template <>
__device__ __forceinline__ __bf16 elem<__bf16>(const uint4& x, int j) {
  const unsigned w = j < 2 ? x.x : j < 4 ? x.y : j < 6 ? x.z : x.w;
  const unsigned short b = (unsigned short)((j & 1) ? (w >> 16) : (w & 0xffffu));
  return __builtin_bit_cast(__bf16, b);
}
template <>
__device__ __forceinline__ float elem<float>(const uint4& x, int j) {
  const unsigned w = j == 0 ? x.x : j == 1 ? x.y : j == 2 ? x.z : x.w;
  return __uint_as_float(w);
}

template <typename T>
struct PrepArgs {
  const T *q, *k, *a, *b;
  const float *A_log, *dt_bias;
  int N, Hk, Hv, r;
  int64_t T_tot, slots;
  float scale, l2_eps;
  const int32_t* cu;
  T *tb, *mp;
  float* scal;
  // with the layer's conv fused (prep_kernel<T, W>, W >= 1): the pre-conv
  // rows and taps, and where the post-conv q, k and v go (q, k above are
  // then not read)
  PrepConv cv;
  T *qo, *ko, *vo;
};

// Causal conv (W taps) + SiLU of 8 channels from W consecutive rows x[0..W)
// (oldest first) held in registers; bf16 result.  wp: the 8 x W taps as
// stored (8 W bf16, channel-major), kept packed until used.
template <int W>
__device__ __forceinline__ uint4 conv_rows(const uint4 (&wp)[W], const uint4* x) {
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const bf16x8 xv = __builtin_bit_cast(bf16x8, x[j]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int flat = e * W + j;
      const float wf = (float)__builtin_bit_cast(bf16x8, wp[flat / 8])[flat % 8];
      acc[e] += wf * (float)xv[e];
    }
  }
  bf16x8 y;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (__bf16)silu_fast(acc[e]);
  return __builtin_bit_cast(uint4, y);
}

template <typename T>
struct PrepSmem {
  static constexpr int kLd = 128 + 16 / (int)sizeof(T);  // row pad of 16 B
  static constexpr int kLdf = 68;  // fp32 64x64 rows, 16-byte aligned
  union {
    struct {
      T Ks[kChunk][kLd];
      T Qs[kChunk][kLd];
    } in;  // raw rows, until the Gram products are done
    struct {
      float Am[kChunk][kLdf];  // A (strictly lower)
      float Tm[kChunk][kLdf];  // (I + A)^{-1}, blocks on and below the diagonal
    } inv;
  } u;
  // in-chunk prefix sums of the log-decay (fp64, see below); every
  // per-token array is read as 16-byte vectors
  alignas(16) double gam[kChunk];
  alignas(16) float bet[kChunk];
  alignas(16) float rk[kChunk];
  alignas(16) float rq[kChunk];
};

__device__ __forceinline__ int scal_index(int t) {
  return 16 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3);
}

// A operand of a Gram product: rows 16i..16i+15 of a staged row block,
// contraction over dk 32kb..32kb+31 in the natural map (value j of lane
// group g at dk 32kb + 8g + j).  The B operand (the other factor's rows) is
// read the same way.
template <typename T>
__device__ __forceinline__ Frag<T> row_frag(const T (*X)[PrepSmem<T>::kLd], int i, int kb,
                                            int lane) {
  return *reinterpret_cast<const Frag<T>*>(&X[16 * i + (lane & 15)][32 * kb + 8 * (lane >> 4)]);
}

// One 16x16 tile X[16i.., :] * Y[16j.., :]^T over dk = 128.
template <typename T>
__device__ __forceinline__ f32x4 gram_tile(const T (*X)[PrepSmem<T>::kLd], int i,
                                           const T (*Y)[PrepSmem<T>::kLd], int j, int lane) {
  f32x4 acc = zero4();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) mma(acc, row_frag<T>(X, i, kb, lane), row_frag<T>(Y, j, kb, lane));
  return acc;
}

// acc += X[ra.., ca..] (16x16) * Y[rb.., cb..] (16x16) with fp32 MFMA,
// contraction index 4kk + g for MFMA kk.
__device__ __forceinline__ void mma16_f32(f32x4& acc, const float (*X)[PrepSmem<float>::kLdf],
                                          int ra, int ca,
                                          const float (*Y)[PrepSmem<float>::kLdf], int rb,
                                          int cb, int m, int g) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[ra + m][ca + 4 * kk + g],
                                               Y[rb + 4 * kk + g][cb + m], acc, 0, 0, 0);
}

// One block per (chunk slot, value head): the chunk's q/k rows and their
// norms, the gates of this value head and their in-chunk prefix sum, the
// Gram products, then A, MP and Tb = (I + A)^{-1} diag(beta), written as
// packed MFMA fragments with the per-token scalars.  CW >= 1 (bf16): the
// q/k rows come from the layer's conv of width CW applied here to the
// pre-conv rows, and the block also writes the post-conv rows: q and k (the
// first value head of each key head) and its value head's v.
template <typename T, int CW>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs<T> p) {
  extern __shared__ __align__(16) char smem_raw[];
  using SM = PrepSmem<T>;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  int c, h;  // workspace slot, value head
  if (!slot_head(blockIdx.x, p.Hk, p.r, p.slots, c, h)) return;
  const int kh = h / p.r;
  // the sequence owning slot c: the largest n with slot_base(n) <= c
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_base(p.cu, p.T_tot, mid) <= c)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int n = lo;
  int64_t s0, s1;
  seq_range(p.cu, p.T_tot, n, s0, s1);
  const int64_t jc = c - (s0 / kChunk + n);
  if (jc < 0 || jc * kChunk >= s1 - s0) return;  // unused slot
  const int64_t t0 = s0 + jc * kChunk;
  const int L = (int)min((int64_t)kChunk, s1 - t0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform branches
  const int g = lane >> 4, m = lane & 15;

  // 1. q and k rows (zero past the sequence end) and their inverse norms,
  //    reduced across the lanes holding one row; the gate inputs (wave 0,
  //    lane = token)
  {
    constexpr int kVec = 16 / sizeof(T);
    constexpr int kPieces = kHeadDim / kVec;  // lanes per row
    constexpr int kRowsPerPass = 256 / kPieces;
    constexpr int kPasses = kChunk / kRowsPerPass;
    const int pc = tid % kPieces, r0 = tid / kPieces;
    // the gate inputs first, loaded by every wave with the token clamped
    // into the chunk (no branch, so nothing waits for them yet): wave 0
    // forms the gates and their prefix sum while the q/k rows are in flight
    const int64_t gidx = (t0 + min(lane, L - 1)) * p.Hv + h;
    const T araw = p.a[gidx], braw = p.b[gidx];
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the q/k rows
    // rows clamped into the chunk, so every load is unconditional and the
    // waits stay exact; rows past the sequence end are zeroed where used
    uint4 kv[kPasses], qv[kPasses];
    if constexpr (CW == 0) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i) {
        const int rr = min(r0 + i * kRowsPerPass, L - 1);
        const int64_t off = ((t0 + rr) * p.Hk + kh) * kHeadDim + pc * kVec;
        kv[i] = *reinterpret_cast<const uint4*>(p.k + off);
        qv[i] = *reinterpret_cast<const uint4*>(p.q + off);
      }
    } else {
      // q | k | v channels of this piece in the pre-conv rows.  Here the
      // thread's rows are kPasses consecutive ones (see row_of), so their
      // taps share rows: CW - 1 + kPasses rows per channel group, all loaded
      // before any is used.
      const int Wq = p.Hk * kHeadDim;
      const int chq = kh * kHeadDim + pc * kVec, chk = Wq + chq;
      const int chv = 2 * Wq + h * kHeadDim + pc * kVec;
      constexpr int R = CW - 1 + kPasses;
      const int64_t tb = t0 + kPasses * r0 - (CW - 1);  // first tap row
      const __bf16* x = static_cast<const __bf16*>(p.cv.x);
      const __bf16* hin = static_cast<const __bf16*>(p.cv.hin);
      // the R tap rows of channels [ch, ch + 8): rows past the chunk are
      // clamped into it (their results are not used); rows before the
      // sequence read its history, or zeros
      auto rows = [&](int ch, uint4 (&xr)[R]) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const int64_t tj = min(tb + j, t0 + L - 1);
          const __bf16* src = nullptr;
          if (tj >= s0)
            src = x + tj * p.cv.ldx + ch;
          else if (hin)
            src = hin + ((int64_t)n * (CW - 1) + (CW - 1) - (s0 - tj)) * p.cv.C + ch;
          xr[j] = src ? *reinterpret_cast<const uint4*>(src) : uint4{0u, 0u, 0u, 0u};
        }
      };
      auto taps = [&](int ch, uint4 (&wp)[CW]) {
        const uint4* w = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(p.cv.w) +
                                                        (int64_t)ch * CW);
#pragma unroll
        for (int u = 0; u < CW; ++u) wp[u] = w[u];
      };
      const bool writes_qk = h % p.r == 0;
      {
        uint4 xq[R], xk[R], wq[CW], wk[CW];
        rows(chq, xq);
        rows(chk, xk);
        taps(chq, wq);
        taps(chk, wk);
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
          const int rr = kPasses * r0 + i;
          qv[i] = conv_rows<CW>(wq, xq + i);
          kv[i] = conv_rows<CW>(wk, xk + i);
          if (rr < L && writes_qk) {
            *reinterpret_cast<uint4*>(p.qo + (t0 + rr) * (int64_t)Wq + chq) = qv[i];
            *reinterpret_cast<uint4*>(p.ko + (t0 + rr) * (int64_t)Wq + chq) = kv[i];
          }
        }
      }
      {
        uint4 xv[R], wv[CW];
        rows(chv, xv);
        taps(chv, wv);
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
          const int rr = kPasses * r0 + i;
          const uint4 vv = conv_rows<CW>(wv, xv + i);
          if (rr < L)
            *reinterpret_cast<uint4*>(p.vo + (t0 + rr) * (int64_t)p.Hv * kHeadDim +
                                      h * kHeadDim + pc * kVec) = vv;
        }
      }
    }
    if (w == 0) {
      float gg = 0.f, bb = 0.f;
      if (lane < L) {
        const float x = to_f32(araw) + p.dt_bias[h];
        const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
        gg = -expf(p.A_log[h]) * sp;
        bb = 1.f / (1.f + expf(-to_f32(braw)));
      }
      // The decays are exponentials of differences gamma_t - gamma_s of
      // prefix sums.  In fp32 such a difference carries an absolute error
      // of an ulp of |gamma| (3e-5 at |gamma| ~ 300, reached within one
      // chunk of strongly decaying heads), a relative error of every factor
      // e^{gamma_t - gamma_s} however small t - s.  Summed in fp64, the
      // differences carry only the rounding of the g they add up.
      const double gs = wave_prefix_sum((double)gg);
      sm.gam[lane] = gs;
      sm.bet[lane] = bb;
    }
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const int rr = CW ? kPasses * r0 + i : r0 + i * kRowsPerPass;
      if (rr >= L) kv[i] = qv[i] = uint4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4*>(&sm.u.in.Ks[rr][pc * kVec]) = kv[i];
      *reinterpret_cast<uint4*>(&sm.u.in.Qs[rr][pc * kVec]) = qv[i];
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const float kx = to_f32(elem<T>(kv[i], e)), qx = to_f32(elem<T>(qv[i], e));
        sk += kx * kx;
        sq += qx * qx;
      }
      // (a row's pieces sit in one 16-lane row of the wave, or two for fp32)
      sk = row16_sum(sk);
      sq = row16_sum(sq);
      if constexpr (kPieces == 32) {
        sk += __shfl_xor(sk, 16);
        sq += __shfl_xor(sq, 16);
      }
      static_assert(kPieces == 16 || kPieces == 32, "row pieces per DPP row");
      // rows past the sequence end get 0, so every product and per-token
      // scalar of theirs is 0 whatever eps is
      if (pc == 0) {
        sm.rk[rr] = rr < L ? rsqrt_fast(sk + p.l2_eps) : 0.f;
        sm.rq[rr] = rr < L ? p.scale * rsqrt_fast(sq + p.l2_eps) : 0.f;
      }
    }
  }
  __syncthreads();

  // per-token scalars; token t = 16T + 4G + R is stored at 16G + 4T + R,
  // so the 16 tokens a lane of lane group G meets in C-layout tiles are
  // contiguous
  if (w == 0) {
    const int t = lane;
    const double gg = sm.gam[t], gL = sm.gam[kChunk - 1];
    const float eg = expf((float)gg);
    float* sc = p.scal + ((int64_t)c * p.Hv + h) * (kScalars * kChunk);
    const int si = scal_index(t);
    sc[si] = eg * sm.rk[t];
    sc[kChunk + si] = expf((float)(gL - gg)) * sm.rk[t];
    sc[2 * kChunk + si] = eg * sm.rq[t];
    sc[3 * kChunk + si] = expf((float)gL);
  }

  // 2. Gram tiles.  Wave w: P^T = K Q^T tiles (a, w) for a <= w (the MP
  //    fragments of query tile w) and G = K K^T tiles (3 - w, j) for
  //    j <= 3 - w; five tiles per wave.
  //    Every wave needs all four k tiles (P: a <= w, G: j <= 3 - w), so each
  //    is read once and meets the wave's q tile w and k tile 3 - w.
  f32x4 pt[4], gt[4];
  const int gi = 3 - w;
  {
    Frag<T> qw[4], kg[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      qw[kb] = row_frag<T>(sm.u.in.Qs, w, kb, lane);
      kg[kb] = row_frag<T>(sm.u.in.Ks, gi, kb, lane);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Frag<T> kt[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kt[kb] = row_frag<T>(sm.u.in.Ks, t, kb, lane);
      pt[t] = zero4();
      gt[t] = zero4();
      if (t <= w)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(pt[t], kt[kb], qw[kb]);
      if (t <= gi)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(gt[t], kg[kb], kt[kb]);
    }
  }
  // decays and norms, in registers.  Every per-token value a lane needs is
  // read first (16-byte reads for the four consecutive tokens 4g..4g+3 of
  // a tile), then each entry is scaled without a branch: the exponent is
  // clamped at 0, which changes nothing on or below the diagonal, and the
  // entries above it are selected to zero.
  {
    // MP^T[s][t] = e^{gamma_t - gamma_s} rq_t rk_s P^T[s][t] for s <= t;
    // lane (g, m) holds s = 16a + 4g + rr, t = 16w + m
    const int t = 16 * w + m;
    const double gt_ = sm.gam[t];
    const float rqt = sm.rq[t];
    double gs[4][4];
    float rks[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const double2 g01 = *reinterpret_cast<const double2*>(&sm.gam[16 * a + 4 * g]);
      const double2 g23 = *reinterpret_cast<const double2*>(&sm.gam[16 * a + 4 * g + 2]);
      const float4 r4 = *reinterpret_cast<const float4*>(&sm.rk[16 * a + 4 * g]);
      gs[a][0] = g01.x; gs[a][1] = g01.y; gs[a][2] = g23.x; gs[a][3] = g23.y;
      rks[a][0] = r4.x; rks[a][1] = r4.y; rks[a][2] = r4.z; rks[a][3] = r4.w;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int s = 16 * a + 4 * g + rr;
        const float v = __expf(fminf((float)(gt_ - gs[a][rr]), 0.f)) * rqt * rks[a][rr] * pt[a][rr];
        pt[a][rr] = s <= t ? v : 0.f;
      }
    // A[t][s] = beta_t e^{gamma_t - gamma_s} rk_t rk_s G[t][s] for t > s;
    // lane (g, m) holds t = 16gi + 4g + rr, s = 16j + m
    const double2 gt01 = *reinterpret_cast<const double2*>(&sm.gam[16 * gi + 4 * g]);
    const double2 gt23 = *reinterpret_cast<const double2*>(&sm.gam[16 * gi + 4 * g + 2]);
    const float4 bt4 = *reinterpret_cast<const float4*>(&sm.bet[16 * gi + 4 * g]);
    const float4 rkt4 = *reinterpret_cast<const float4*>(&sm.rk[16 * gi + 4 * g]);
    const double gtv[4] = {gt01.x, gt01.y, gt23.x, gt23.y};
    const float btk[4] = {bt4.x * rkt4.x, bt4.y * rkt4.y, bt4.z * rkt4.z, bt4.w * rkt4.w};
    double gsj[4];
    float rksj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gsj[j] = sm.gam[16 * j + m];
      rksj[j] = sm.rk[16 * j + m];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 16 * j + m;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int t = 16 * gi + 4 * g + rr;
        const float v = btk[rr] * __expf(fminf((float)(gtv[rr] - gsj[j]), 0.f)) * rksj[j] * gt[j][rr];
        gt[j][rr] = t > s ? v : 0.f;
      }
    }
  }
  // MP fragments (query tile w, k-groups 0 and 1): two stacked P^T tiles
  // are exactly the B operand of the output product
  {
    T* dst = p.mp + ((int64_t)c * p.Hv + h) * (kTbFrags * kFragElems);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = pt[2 * kb][j];
        x[4 + j] = pt[2 * kb + 1][j];
      }
      if (!zero_frag_index(2 * w + kb)) store_packed(dst + (2 * w + kb) * kFragElems + lane * 8, x);
    }
  }
  __syncthreads();  // q/k rows are dead from here; Am/Tm reuse their space
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j <= gi)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sm.u.inv.Am[16 * gi + 4 * g + rr][16 * j + m] = gt[j][rr];
  __syncthreads();

  // 3. (I + A)^{-1}: diagonal 16x16 blocks by forward substitution (wave w
  //    owns block w, lane = column), column by column so the row updates of
  //    one step are independent; entries above the diagonal come out 0
  if (lane < 16) {
    const int b0 = 16 * w, cc = lane;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = rr == cc ? 1.f : 0.f;
#pragma unroll
    for (int s = 0; s < 15; ++s)
#pragma unroll
      for (int rr = s + 1; rr < 16; ++rr) x[rr] -= sm.u.inv.Am[b0 + rr][b0 + s] * x[s];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sm.u.inv.Tm[b0 + rr][b0 + cc] = x[rr];
  }
  __syncthreads();
  // ... then block (i, j), i > j, by distance d = i - j:
  //     T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj
  // (fp32 MFMA, one wave per block; the sum stays in registers as the B
  // operand of the second product, with contraction index 4g + kk)
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int j = w, i = w + d;
      f32x4 xs = zero4();
#pragma unroll
      for (int e = 0; e < d; ++e)
        mma16_f32(xs, sm.u.inv.Am, 16 * i, 16 * (j + e), sm.u.inv.Tm, 16 * (j + e), 16 * j, m, g);
      f32x4 y = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.u.inv.Tm[16 * i + m][16 * i + 4 * g + kk],
                                                 xs[kk], y, 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sm.u.inv.Tm[16 * i + 4 * g + rr][16 * j + m] = -y[rr];
    }
    __syncthreads();
  }

  // 4. Tb = T diag(beta) as A-operand fragments [token t][token s]: wave w
  //    writes token tile w (k-groups 0, 1); blocks above the diagonal are 0
  {
    T* dst = p.tb + ((int64_t)c * p.Hv + h) * (kTbFrags * kFragElems);
    const int t = 16 * w + m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float x[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int s = 32 * kb + 16 * half + 4 * g;
        if (2 * kb + half <= w) {
          const float4 tv = *reinterpret_cast<const float4*>(&sm.u.inv.Tm[t][s]);
          const float4 bv = *reinterpret_cast<const float4*>(&sm.bet[s]);
          x[4 * half + 0] = tv.x * bv.x;
          x[4 * half + 1] = tv.y * bv.y;
          x[4 * half + 2] = tv.z * bv.z;
          x[4 * half + 3] = tv.w * bv.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * half + e] = 0.f;
        }
      }
      if (!zero_frag_index(2 * w + kb)) store_packed(dst + (2 * w + kb) * kFragElems + lane * 8, x);
    }
  }
}

// --------------------------------------------------------------- chain ----

template <typename T>
struct ChainArgs {
  const T *k, *v;
  const float* state_in;
  float* state_out;
  int N, Hk, Hv, r;
  int64_t T_tot;
  const int32_t* cu;
  const T* tb;
  const float* scal;
  T *hc, *vp;  // exported state at chunk entry / delta writes, as fragments
  // Sequence-parallel scan of one sequence (seg_mode 0: one pass over each
  // sequence).  The sequence's chunks form nseg segments of seg_chunks.
  // seg_mode 1 (pass A): segment g = 0 runs from state_in with its exports
  // and leaves its final state in seg_S[1]; each segment 1 <= g <= nseg - 2
  // runs twice, from H = 0 (part 1, final state to seg_B[g]) and from H = I
  // with v taken as zero (part 2, final state to seg_M[g]): the segment's
  // affine map H -> M H + B.  seg_mode 2 (pass C): each segment g >= 1 runs
  // from seg_S[g] with its exports; the last segment writes state_out.  The
  // (part, segment, value head) runs take the place of the value heads in
  // the block numbering, so they spread over the XCDs as heads do.  seg_S[g] for g >= 2 comes from
  // scan_combine_kernel between the two.  Buffers are [nseg][N Hv][128][128]
  // fp32 in the state layout.
  int seg_mode, seg_chunks, nseg;
  float *seg_S, *seg_B, *seg_M;
};

// A staged chunk of k rows keeps each 256-byte (bf16) or 512-byte (fp32)
// row whole, with its 16-byte units permuted: position pos of row r holds
// unit pos ^ kswz(r).  Eight consecutive rows at one column, and the 4 x 4
// (row, unit) pattern of a transposed read, then fall into distinct banks.
__device__ __forceinline__ int kswz(int row) {
  return 4 * (row & 3) + ((row >> 2) & 3);
}

// Element offset of k[row][col] in a staged chunk.
template <typename T>
__device__ __forceinline__ int k_off(int row, int col) {
  constexpr int kVec = 16 / (int)sizeof(T);
  return row * kHeadDim + (((col / kVec) ^ kswz(row)) * kVec) + (col % kVec);
}

// Compute units of the device (gfx950: 256): a chain grid up to this size
// runs one block per CU.
constexpr int64_t kChainCUs = 256;

// One staged chunk of the chain's operands.
template <typename T>
struct ChainStage {
  T K[kChunk * kHeadDim];        // k rows (units permuted, see kswz)
  T Tb[kTbFrags * kFragElems];   // packed Tb fragments
  T V[kChunk * kDvBlock];        // v[token][16 columns of the block]
  float sc[kScalars * kChunk];   // ek, fk, fq, e^{gamma_L}
};

// NS staging slots: bf16 four (three chunks in flight beyond the current
// one, 116 KB, one block per CU), two (62 KB, two blocks per CU) or one
// (35 KB, four blocks per CU; the next chunk is staged only once the
// current one is done); fp32 stages are twice as large and two fit
template <typename T, int NS>
struct ChainSmem {
  static constexpr int kSlots = NS;
  using Stage = ChainStage<T>;
  Stage st[kSlots];
  T Hx[4 * kFragElems];  // H (state at chunk entry) as B operand over dk
  T Rx[2 * kFragElems];  // R as B operand over tokens
  T Wx[2 * kFragElems];  // diag(fk) V' as B operand over tokens
};

// Global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// lds_base + 16 l (lds_base wave-uniform); counted by vmcnt.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(
      src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Copies issued per staged chunk (1 KB each): the stage less Tb's two
// zero fragments.
template <typename T>
constexpr int chunk_copies() {
  return (int)(sizeof(ChainStage<T>) / 1024) -
         2 * kFragElems * (int)sizeof(T) / 1024;
}

// Stages chunks into LDS slots with direct copies (one wave).  Rows past
// the sequence end repeat its last row, so every copy reads inside the
// tensors; their per-token scalars are zero (see prep), so they add nothing.
// Each lane's byte offsets of its k and v pieces within a full chunk are
// fixed for the whole pass and computed once, so a full chunk's copies are
// a wave-uniform base plus those offsets (no per-copy address arithmetic on
// the SIMD it shares with a chain wave).
template <typename T>
struct ChunkCopier {
  static constexpr int kVec = 16 / (int)sizeof(T);
  static constexpr int kRowUnits = kHeadDim / kVec;
  static constexpr int kKCopies = kChunk * kRowUnits / 64;
  static constexpr int kVUnits = kDvBlock / kVec;
  static constexpr int kVCopies = kChunk * kVUnits / 64;
  static constexpr int kTbCopies = kTbFrags * kFragElems / kVec / 64;
  static_assert(sizeof(ChainStage<T>) ==
                    (size_t)(kKCopies + kTbCopies + kVCopies + 1) * 1024,
                "stage regions must be whole 1 KB copies");
  uint32_t koff[kKCopies], voff[kVCopies], o16;

  __device__ __forceinline__ void init(const ChainArgs<T>& p, int lane, int dvb) {
    const uint32_t rs = (uint32_t)p.Hk * kHeadDim * sizeof(T);
    const uint32_t vrs = (uint32_t)p.Hv * kHeadDim * sizeof(T);
    o16 = 16u * lane;
#pragma unroll
    for (int i = 0; i < kKCopies; ++i) {
      const int P = 64 * i + lane, row = P / kRowUnits, pos = P % kRowUnits;
      koff[i] = row * rs + (uint32_t)((pos ^ kswz(row)) * 16);
    }
#pragma unroll
    for (int i = 0; i < kVCopies; ++i) {
      const int P = 64 * i + lane, row = P / kVUnits, pc = P % kVUnits;
      voff[i] = row * vrs + (uint32_t)((dvb * kDvBlock + pc * kVec) * sizeof(T));
    }
  }

  // part 0: the k rows; part 1: v, Tb and the scalars; 2: all
  __device__ __forceinline__ void copy(const ChainArgs<T>& p,
                                       ChainStage<T>& st, int lane,
                                       int64_t slot, int64_t t0, int L, int h, int kh,
                                       int dvb, int part = 2) {
    const char* kb = reinterpret_cast<const char*>(p.k + (t0 * p.Hk + kh) * kHeadDim);
    const char* vb = reinterpret_cast<const char*>(p.v + (t0 * p.Hv + h) * kHeadDim);
    const bool do_k = part != 1, do_rest = part != 0;
    if (L == kChunk) {
      // (each 32-bit offset is made opaque in place, so that its widening
      // is not hoisted out of the chunk loop as a 64-bit vector value: a
      // scalar base plus a widened 32-bit offset is the copy's scalar-base
      // address form, with no vector instruction per copy)
      if (do_k) {
#pragma unroll
        for (int i = 0; i < kKCopies; ++i) {
          asm volatile("" : "+v"(koff[i]));
          dma16(kb + koff[i], st.K + 64 * i * kVec);
        }
      }
      if (do_rest) {
#pragma unroll
        for (int i = 0; i < kVCopies; ++i) {
          asm volatile("" : "+v"(voff[i]));
          dma16(vb + voff[i], st.V + 64 * i * kVec);
        }
      }
    } else {
      const int64_t rs = (int64_t)p.Hk * kHeadDim * sizeof(T);
      const int64_t vrs = (int64_t)p.Hv * kHeadDim * sizeof(T);
      if (do_k) {
#pragma unroll
        for (int i = 0; i < kKCopies; ++i) {
          const int P = 64 * i + lane, row = P / kRowUnits, pos = P % kRowUnits;
          dma16(kb + min(row, L - 1) * rs + (pos ^ kswz(row)) * 16, st.K + 64 * i * kVec);
        }
      }
      if (do_rest) {
#pragma unroll
        for (int i = 0; i < kVCopies; ++i) {
          const int P = 64 * i + lane, row = P / kVUnits, pc = P % kVUnits;
          dma16(vb + min(row, L - 1) * vrs + (dvb * kDvBlock + pc * kVec) * (int)sizeof(T),
                st.V + 64 * i * kVec);
        }
      }
    }
    if (!do_rest) return;
    // Tb and the gates: lane l's 16 bytes of each 1 KB copy (scalar base
    // plus the one opaque lane offset, as above)
    const char* tb = reinterpret_cast<const char*>(
        p.tb + (slot * p.Hv + h) * (kTbFrags * kFragElems));
    const char* sc = reinterpret_cast<const char*>(
        p.scal + (slot * p.Hv + h) * (kScalars * kChunk));
    asm volatile("" : "+v"(o16));
    constexpr int kFragCopies = kFragElems / kVec / 64;
#pragma unroll
    for (int i = 0; i < kTbCopies; ++i) {
      if (zero_frag_index(i / kFragCopies)) continue;
      // (the copy's scalar base is opaque too, or its constant part is
      // folded into a vector address)
      const char* bi = tb + 1024 * i;
      asm volatile("" : "+s"(bi));
      dma16(bi + o16, st.Tb + 64 * i * kVec);
    }
    dma16(sc + o16, st.sc);
  }
};

// Waits until at most n chunks' copies are still in flight (n = 0, 1, 2).
template <typename T>
__device__ __forceinline__ void wait_copies(int n) {
  constexpr int D = chunk_copies<T>();
  // s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and
  // lgkmcnt 11:8 left at their maxima
  constexpr int kRest = (0x7 << 4) | (0xf << 8);
  constexpr int kVm1 = D < 64 ? D : 63, kVm2 = 2 * D < 64 ? 2 * D : 63;
  static_assert(sizeof(T) == 4 || 2 * D < 64, "copies in flight exceed vmcnt");
  asm volatile("" ::: "memory");
  if (n <= 0)
    __builtin_amdgcn_s_waitcnt(kRest);
  else if (n == 1)
    __builtin_amdgcn_s_waitcnt(kRest | (kVm1 & 15) | ((kVm1 >> 4) << 14));
  else
    __builtin_amdgcn_s_waitcnt(kRest | (kVm2 & 15) | ((kVm2 >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Workgroup barrier for the loader wave, which writes LDS only through
// direct copies and waits for them itself: no fence, so the compiler adds
// no waits for copies still in flight.
__device__ __forceinline__ void plain_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A operand of the state update for tile t of chain wave w (state rows
// dk = 32w + 8(i/4) + 4t + i%4 for lane row i) and tokens 32kb..32kb+31:
// value j of lane (G, i) is k[32kb + perm(G, j)][dk].
template <typename T>
__device__ __forceinline__ Frag<T> kt_frag(const T* K, int w, int t, int kb, int lane);

template <>
__device__ __forceinline__ Frag<__bf16> kt_frag<__bf16>(const __bf16* K, int w, int t,
                                                        int kb, int lane) {
  // ds_read_b64_tr_b16: in each 16-lane group, result lane i takes element
  // i%4 of the 8 bytes addressed by source lane 4j + i/4, for j = 0..3.
  // Source lane (G, 4j+q) addresses k[32kb + 4G + j][32w + 8q + 4t..+3]
  // (and the row 16 further for values 4..7).
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int G = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
  const int col = 32 * w + 8 * q + 4 * t;
  const __bf16* a0 = K + k_off<__bf16>(32 * kb + 4 * G + j, col);
  const __bf16* a1 = K + k_off<__bf16>(32 * kb + 16 + 4 * G + j, col);
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) void*)(a0));
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) void*)(a1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 both = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  Frag<__bf16> f;
  f.v = __builtin_bit_cast(bf16x8, both);
  return f;
}

template <>
__device__ __forceinline__ Frag<float> kt_frag<float>(const float* K, int w, int t,
                                                      int kb, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int dk = 32 * w + 8 * (i >> 2) + 4 * t + (i & 3);
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = K[k_off<float>(32 * kb + kperm(g, j), dk)];
  return f;
}

// The four staged v values of lane (g, m) of chain wave w: v[16w + 4g + j][m]
// for j = 0..3 (the accumulator rows of its token tile), as one transposed
// 8-byte read for bf16.  Source lane (G, 4j + q) addresses columns
// 4q..4q+3 of row 16w + 4G + j; result lane m takes element m % 4 of source
// lane 4j + m / 4, which is column m.
template <typename T>
__device__ __forceinline__ void v_col4(const T* V, int w, int lane, float (&v)[4]);

template <>
__device__ __forceinline__ void v_col4<__bf16>(const __bf16* V, int w, int lane,
                                               float (&v)[4]) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int G = lane >> 4, s = lane & 15;
  const __bf16* a = V + (16 * w + 4 * G + (s >> 2)) * kDvBlock + 4 * (s & 3);
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) void*)(a));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    v[j] = __uint_as_float((unsigned)(unsigned short)r[j] << 16);
}

template <>
__device__ __forceinline__ void v_col4<float>(const float* V, int w, int lane,
                                              float (&v)[4]) {
  const int g = lane >> 4, m = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = V[(16 * w + 4 * g + j) * kDvBlock + m];
}

// A operand of Y = K H for token rows 16w..16w+15 and dk 32kb..32kb+31: value
// j of lane (g, m) is k[16w + m][32kb + 8g + j].
template <typename T>
__device__ __forceinline__ Frag<T> k_frag(const T* K, int w, int kb, int lane) {
  const int g = lane >> 4, m = lane & 15, row = 16 * w + m;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const Frag<T>*>(K + k_off<T>(row, 32 * kb + 8 * g));
  } else {
    const float4 lo = *reinterpret_cast<const float4*>(K + k_off<T>(row, 32 * kb + 8 * g));
    const float4 hi = *reinterpret_cast<const float4*>(K + k_off<T>(row, 32 * kb + 8 * g + 4));
    Frag<T> f;
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
}

// Writes one 16-row accumulator tile into its half of a B-operand fragment
// buffer (k-group = tile / 2, half = tile % 2).
template <typename T>
__device__ __forceinline__ void put_half(T* buf, int tile, int lane, const f32x4& x) {
  T* dst = buf + (tile >> 1) * kFragElems + lane * 8 + 4 * (tile & 1);
  const float y[4] = {x[0], x[1], x[2], x[3]};
  store4(dst, y);  // one 8-byte (bf16) or 16-byte (fp32) write
}

// One block owns 16 value columns of one (sequence, value head) state.
// Chain waves 0-3 split every per-chunk product by rows: wave w owns token
// rows 16w..16w+15 of Y = K H, R and V' = Tb R, and the state rows
// dk = 32w + 8g + 4t + rr (lane group g, tile t, accumulator row rr) of the
// update -- an assignment under which two stacked state tiles are the B
// operand over dk with value j of lane group g at dk 32w + 8g + j, so the k
// rows are read in their natural order.  R, diag(fk) V' and the new state
// are exchanged through LDS (three barriers per chunk); each phase issues
// its reads of the staged chunk together with its exchange reads.  Wave 4
// stages chunks into a ring of LDS slots with direct copies, up to three
// chunks ahead.  The chain waves also export the state at chunk entry and
// V' (fragments) for the output kernel.  Block ids put the 8 column blocks
// of a head on one XCD (same blockIdx % 8), so they share its L2 for the k
// rows and Tb.
template <typename T, int NS>
__global__ __launch_bounds__(320) void chain_kernel(ChainArgs<T> p) {
  extern __shared__ __align__(1024) char smem_raw[];
  using SM = ChainSmem<T, NS>;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  constexpr int S = SM::kSlots;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, s8 = bid >> 3;
  const int vu = (s8 >> 3) * 8 + xcd;  // a value head, or a scan run
  const int dvb = s8 & 7;
  const int units = p.N * p.Hv;
  int unit = vu, part = 0, sg = 0;
  if (p.seg_mode == 1) {
    if (vu >= units * (2 * p.nseg - 3)) return;  // block-uniform: every wave leaves
    if (vu >= units) {
      const int j = vu - units, pair = j / units;
      unit = j % units;
      sg = 1 + pair / 2;
      part = 1 + pair % 2;
    }
  } else if (p.seg_mode == 2) {
    if (vu >= units * (p.nseg - 1)) return;
    unit = vu % units;
    sg = 1 + vu / units;
  } else if (unit >= units) {
    return;
  }
  // block-uniform; the divisions expand to vector code, so their results are
  // moved back to scalar registers, which keeps every copy address a
  // scalar base plus a fixed per-lane offset (no per-copy vector adds)
  const int n = __builtin_amdgcn_readfirstlane(unit / p.Hv);
  const int h = __builtin_amdgcn_readfirstlane(unit % p.Hv);
  const int kh = __builtin_amdgcn_readfirstlane(h / p.r);
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform, so that the branches on it (the state export) are scalar
  // and no matrix instruction runs under a partial or empty lane mask
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, m = lane & 15;
  const int dv = dvb * kDvBlock + m;

  int64_t s0, s1;
  seq_range(p.cu, p.T_tot, n, s0, s1);
  const int nch = (int)((s1 - s0 + kChunk - 1) / kChunk);
  const int64_t slot0 = s0 / kChunk + n;
  auto chunk_L = [&](int i) {
    return (int)min((int64_t)kChunk, s1 - s0 - (int64_t)i * kChunk);
  };
  // this block's chunks [cb, cb + nloc), its start and end states, and
  // whether it runs the true sequence (exports) or a segment map part
  int cb = 0, nloc = nch;
  const size_t sbase = ((size_t)unit * kHeadDim + dv) * kHeadDim;
  const float* h_in = p.state_in;
  float* h_out = p.state_out;
  if (p.seg_mode) {
    cb = min(sg * p.seg_chunks, nch);
    nloc = min(cb + p.seg_chunks, nch) - cb;
    const size_t seg_stride = (size_t)p.N * p.Hv * kHeadDim * kHeadDim;
    if (part == 1) {
      h_in = nullptr;
      h_out = p.seg_B + sg * seg_stride;
    } else if (part == 2) {
      h_in = nullptr;
      h_out = p.seg_M + sg * seg_stride;
    } else if (p.seg_mode == 1) {
      h_out = p.seg_S + seg_stride;  // segment 0 ends where segment 1 starts
    } else {
      h_in = p.seg_S + sg * seg_stride;
      if (sg != p.nseg - 1) h_out = nullptr;
    }
  }
  const bool exports = part == 0;
  const bool v_zero = part == 2;

  if (w < 4) {
    // the chain waves' instructions go first when the loader wave on the
    // same SIMD is also ready
    __builtin_amdgcn_s_setprio(2);
    f32x4 H[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (part == 2) {
        // H = I: state row dk = 32w + 8g + 4t + rr, column dv
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) H[t][rr] = (32 * w + 8 * g + 4 * t + rr == dv) ? 1.f : 0.f;
      } else {
        H[t] = h_in ? *reinterpret_cast<const f32x4*>(h_in + sbase + 32 * w + 8 * g + 4 * t)
                    : zero4();
      }
    }
    {
      // the start state is chunk cb's entry state: this wave exports its
      // k-group of it here, and each later chunk's where phase 3 forms it
      const Frag<T> hx = frag_from_acc_t<T>(H[0], H[1]);
      *reinterpret_cast<Frag<T>*>(&sm.Hx[(w * 64 + lane) * 8]) = hx;
      if (exports && nloc > 0)
        *reinterpret_cast<Frag<T>*>(
            &p.hc[(((slot0 + cb) * p.Hv + h) * kDvBlocks + dvb) * (4 * kFragElems) +
                  (w * 64 + lane) * 8]) = hx;
    }
    // Tb's fragments above the diagonal are never staged: zero them once in
    // every slot, so that each wave's V' = Tb R takes both k-groups with no
    // branch (waves 0 and 1 add a product with zero)
    {
      constexpr int kVec = 16 / (int)sizeof(T);
      constexpr int kUnits = 2 * kFragElems / kVec;  // 16-byte units per slot
#pragma unroll
      for (int u = tid; u < S * kUnits; u += 256) {
        const int sl = u / kUnits, f = (u % kUnits) / (kFragElems / kVec);
        const int e = (u % (kFragElems / kVec)) * kVec;
        *reinterpret_cast<uint4*>(&sm.st[sl].Tb[(2 * f + 1) * kFragElems + e]) =
            uint4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();
    for (int li = 0; li < nloc; ++li) {
      // (one slot: an extra barrier opens each iteration after the first,
      // once the loader has staged its chunk)
      if (S == 1 && li > 0) __syncthreads();
      const int i = cb + li;
      const typename SM::Stage& cs = sm.st[li % S];
      const int64_t fo = ((slot0 + i) * p.Hv + h) * kDvBlocks + dvb;
      T* vp_out = p.vp + fo * (2 * kFragElems);
      // phase 1: Y = K H for token tile w, R = V - diag(ek) Y
      Frag<T> hb[4], kf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        hb[kb] = *reinterpret_cast<const Frag<T>*>(&sm.Hx[(kb * 64 + lane) * 8]);
        kf[kb] = k_frag<T>(cs.K, w, kb, lane);
      }
      // tokens 16w + 4g + rr sit at scal_index = 16g + 4w + rr
      float v[4];
      v_col4<T>(cs.V, w, lane, v);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v[rr] = v_zero ? 0.f : v[rr];
      const f32x4 ek = *reinterpret_cast<const f32x4*>(&cs.sc[16 * g + 4 * w]);
      // phase 2's staged operands (Tb fragments and fk) are read now, behind
      // this phase's reads, so that after the next barrier only the
      // exchanged R is read (token tiles 0 and 1 take Tb's zeroed fragments
      // above the diagonal)
      Frag<T> tbf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        tbf[kb] = *reinterpret_cast<const Frag<T>*>(&cs.Tb[((2 * w + kb) * 64 + lane) * 8]);
      const f32x4 fk = *reinterpret_cast<const f32x4*>(&cs.sc[kChunk + 16 * g + 4 * w]);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 y0 = zero4(), y1 = zero4();
      mma(y0, kf[0], hb[0]);
      mma(y1, kf[1], hb[1]);
      mma(y0, kf[2], hb[2]);
      mma(y1, kf[3], hb[3]);
      f32x4 R;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) R[rr] = v[rr] - ek[rr] * (y0[rr] + y1[rr]);
      put_half<T>(sm.Rx, w, lane, R);
      __syncthreads();
      // phase 2: V' = Tb R for token tile w
      Frag<T> rb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        rb[kb] = *reinterpret_cast<const Frag<T>*>(&sm.Rx[(kb * 64 + lane) * 8]);
      // phase 3's staged operands (k^T fragments of this wave's state rows,
      // e^{gamma_L}), likewise read a phase ahead
      Frag<T> ktf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) ktf[t][kb] = kt_frag<T>(cs.K, w, t, kb, lane);
      const float eL = cs.sc[3 * kChunk];
      // every read goes out before the first product (left to itself the
      // scheduler delays reads behind it)
      __builtin_amdgcn_sched_barrier(0);
      f32x4 Vp = zero4();
      mma(Vp, tbf[0], rb[0]);
      mma(Vp, tbf[1], rb[1]);
      f32x4 Wv;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) Wv[rr] = Vp[rr] * fk[rr];
      put_half<T>(sm.Wx, w, lane, Wv);
      if (exports) put_half<T>(vp_out, w, lane, Vp);
      // the decay of the state rows needs no exchanged value: done before
      // the barrier, so phase 3 starts with its products
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) H[t][rr] *= eL;
      __syncthreads();
      // phase 3: H <- e^{gamma_L} H + K^T diag(fk) V' for this wave's rows
      Frag<T> wb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        wb[kb] = *reinterpret_cast<const Frag<T>*>(&sm.Wx[(kb * 64 + lane) * 8]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        mma(H[t], ktf[t][0], wb[0]);
        mma(H[t], ktf[t][1], wb[1]);
      }
      {
        const Frag<T> hx = frag_from_acc_t<T>(H[0], H[1]);
        *reinterpret_cast<Frag<T>*>(&sm.Hx[(w * 64 + lane) * 8]) = hx;
        // chunk i + 1's entry state
        if (exports && li + 1 < nloc)
          *reinterpret_cast<Frag<T>*>(
              &p.hc[(fo + (int64_t)p.Hv * kDvBlocks) * (4 * kFragElems) + (w * 64 + lane) * 8]) =
              hx;
      }
      __syncthreads();
    }
    if (h_out) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *reinterpret_cast<f32x4*>(h_out + sbase + 32 * w + 8 * g + 4 * t) = H[t];
    }
  } else {
    // Loader wave.  Chunk j goes to slot j % S.  It is issued at the start
    // of iteration j - S + 1, once the chain waves have finished iteration
    // j - S (the slot's previous chunk; every read of it completed before
    // that iteration's last barrier), and waited for before the last
    // barrier of iteration j - 1.  Three barriers per iteration, as the
    // chain waves.
    // (its copies go out ahead of the chain wave on its SIMD; it spends the
    // rest of its time waiting at barriers)
    __builtin_amdgcn_s_setprio(3);
    ChunkCopier<T> cp;
    cp.init(p, lane, dvb);
    // (j counts this block's chunks: its chunk cb + j)
    auto stage = [&](int j, int part = 2) {
      const int i = cb + j;
      cp.copy(p, sm.st[j % S], lane, slot0 + i, s0 + (int64_t)i * kChunk, chunk_L(i), h, kh,
              dvb, part);
    };
    if constexpr (S == 1) {
      // One slot: chunk j + 1 is issued once every read of chunk j is done
      // (after iteration j's last barrier) and waited for before the extra
      // barrier that opens iteration j + 1.
      if (nloc > 0) stage(0);
      wait_copies<T>(0);
      plain_barrier();
      for (int i = 0; i < nloc; ++i) {
        plain_barrier();
        plain_barrier();
        plain_barrier();
        if (i + 1 < nloc) {
          stage(i + 1);
          wait_copies<T>(0);
          plain_barrier();
        }
      }
    } else {
      const int pro = min(S - 1, nloc);  // chunks issued before the first iteration
      for (int j = 0; j < pro; ++j) stage(j);
      wait_copies<T>(pro - 1);  // chunk 0 has landed
      plain_barrier();
      for (int i = 0; i < nloc; ++i) {
        // the chunk's k rows before the first barrier, the rest before the
        // second (all of it is issued before the wait below)
        if (i + S - 1 < nloc) stage(i + S - 1, 0);
        plain_barrier();
        if (i + S - 1 < nloc) stage(i + S - 1, 1);
        plain_barrier();
        if (i + 1 < nloc) wait_copies<T>(min(i + S - 1, nloc - 1) - (i + 1));
        plain_barrier();
      }
    }
  }
}

// ---------------------------------------------------------- scan combine ----

// Start states of the scan's segments, in order, for g = 1 .. nseg - 2.  A
// segment maps its start state H to M H + B.  In the state layout S = H^T
// the runs leave seg_B[g] = B^T and, the M run starting from H = I,
// seg_M[g] = M^T; so S[g + 1] = (M H + B)^T = S[g] seg_M[g] + seg_B[g], a
// plain row-major product.  One block per (value head, 4 state rows): rows
// of S are independent, so a block carries its rows through every segment
// in order with no other block; fp32.
struct CombineArgs {
  float *seg_S;
  const float *seg_B, *seg_M;
  int units, nseg;
};

// M and the rows are double-buffered in LDS.  A step loads its B rows, then
// the next segment's M into registers, applies the current M from LDS, and
// stores the next M into the other buffer: loads complete in issue order, so
// the product waits only for B, and the next M arrives during the product.
// One barrier per step.  A block owns kCombineRows rows of S (each thread
// one column of kCombineRows / 2 rows), so each M is read by 128 /
// kCombineRows blocks per value head.
constexpr int kCombineRows = 2;
struct CombineSmem {
  float M[2][kHeadDim][kHeadDim];
  float rows[2][kCombineRows][kHeadDim];
};

// (one block of four waves per CU: 130 KB of LDS; registers for the
// prefetched M)
__global__ __launch_bounds__(256, 1) void scan_combine_kernel(CombineArgs p) {
  extern __shared__ __align__(16) char smem_raw[];
  CombineSmem& sm = *reinterpret_cast<CombineSmem*>(smem_raw);
  constexpr int R = kCombineRows / 2;  // rows per thread
  const int unit = blockIdx.x, r0 = kCombineRows * blockIdx.y;
  if (unit >= p.units || p.nseg < 3) return;
  const int tid = threadIdx.x, j = tid & 127, rh = (tid >> 7) * R;  // column, first row
  const size_t stride = (size_t)p.units * kHeadDim * kHeadDim;
  const size_t ubase = (size_t)unit * kHeadDim * kHeadDim;
  // thread tid moves 16-byte pieces tid, tid + 256, ... of a 64 KB matrix
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.seg_M + stride + ubase);
    f32x4* dst = reinterpret_cast<f32x4*>(&sm.M[0][0][0]);
    f32x4 x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = src[tid + 256 * i];
    const float* s1 = p.seg_S + stride + ubase;
#pragma unroll
    for (int e = 0; e < R; ++e) sm.rows[0][rh + e][j] = s1[(size_t)(r0 + rh + e) * kHeadDim + j];
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[tid + 256 * i] = x[i];
  }
  __syncthreads();
  for (int sg = 1; sg + 1 < p.nseg; ++sg) {
    const int cur = (sg - 1) & 1;
    const float* B = p.seg_B + sg * stride + ubase;
    float acc[R];
#pragma unroll
    for (int e = 0; e < R; ++e) acc[e] = B[(size_t)(r0 + rh + e) * kHeadDim + j];
    __builtin_amdgcn_sched_barrier(0);  // B's loads go first
    // the next M (at the last step a repeat of the current one, unused):
    // loaded and stored unconditionally, so it stays in registers
    const int nx = min(sg + 1, p.nseg - 2);
    f32x4 x[16];
    {
      const f32x4* src = reinterpret_cast<const f32x4*>(p.seg_M + nx * stride + ubase);
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = src[tid + 256 * i];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 8
    for (int c = 0; c < kHeadDim; ++c) {
      const float mv = sm.M[cur][c][j];
#pragma unroll
      for (int e = 0; e < R; ++e) acc[e] = fmaf(sm.rows[cur][rh + e][c], mv, acc[e]);
    }
    float* out = p.seg_S + (sg + 1) * stride + ubase;
#pragma unroll
    for (int e = 0; e < R; ++e) {
      out[(size_t)(r0 + rh + e) * kHeadDim + j] = acc[e];
      sm.rows[cur ^ 1][rh + e][j] = acc[e];
    }
    {
      f32x4* dst = reinterpret_cast<f32x4*>(&sm.M[cur ^ 1][0][0]);
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[tid + 256 * i] = x[i];
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------- out ----


// Element j of 4 consecutive values held in their input format.
template <typename T>
__device__ __forceinline__ float z_elem(const uint2& x, int j) {
  const unsigned w = j < 2 ? x.x : x.y;
  const unsigned short b = (unsigned short)((j & 1) ? (w >> 16) : (w & 0xffffu));
  return (float)__builtin_bit_cast(__bf16, b);
}
template <typename T>
__device__ __forceinline__ float z_elem(const uint4& x, int j) {
  return __uint_as_float(j == 0 ? x.x : j == 1 ? x.y : j == 2 ? x.z : x.w);
}

template <typename T>
struct OutArgs {
  const T *q, *z;
  const float* norm_w;
  T* o;
  int N, Hk, Hv, r;
  int64_t T_tot, slots;
  float norm_eps;
  const int32_t* cu;
  const T *mp, *hc, *vp;
  const float* scal;
};

template <typename T>
struct OutSmem {
  T Q[kChunk * kHeadDim];       // raw q rows, 16-byte units permuted (kswz)
  T MP[kTbFrags * kFragElems];  // packed MP fragments
  float fq[kChunk];             // scal_index order
  float ss[4][kChunk];          // per-wave partial sums of squares
};

// Outputs of one (chunk, value head), all 128 value columns, computed
// transposed so that each lane holds 4 consecutive columns of a row:
//   O^T = H^T (diag(fq) Q)^T + V'^T MP^T
// The exported state fragments (lane (g, m) holds H[32kb + 8g + j][16 dvb +
// m]) and delta-write fragments (V'[32kb + perm(g, j)][16 dvb + m]) are the A
// operands as they are; q rows (read in natural order) and MP are the B
// operands.  Wave w owns value columns 32w..32w+31 (two exported blocks).
// With z given, the gated RMSNorm of each row is applied before the store
// (row sums of squares combined across lanes and waves).
template <typename T>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 4 : 2) void out_kernel(OutArgs<T> p) {
  extern __shared__ __align__(16) char smem_raw[];
  OutSmem<T>& sm = *reinterpret_cast<OutSmem<T>*>(smem_raw);
  int c, h;  // workspace slot, value head
  if (!slot_head(blockIdx.x, p.Hk, p.r, p.slots, c, h)) return;
  const int kh = h / p.r;
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_base(p.cu, p.T_tot, mid) <= c)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int n = lo;
  int64_t s0, s1;
  seq_range(p.cu, p.T_tot, n, s0, s1);
  const int64_t jc = c - (s0 / kChunk + n);
  if (jc < 0 || jc * kChunk >= s1 - s0) return;  // unused slot
  const int64_t t0 = s0 + jc * kChunk;
  const int L = (int)min((int64_t)kChunk, s1 - t0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: copy bases, branches
  const int g = lane >> 4, m = lane & 15;

  // Every load is issued before anything waits.  fq first (the only
  // staged value that goes through registers), then the q rows and the MP
  // fragments as direct copies into LDS, then this wave's exported
  // fragments and z.  q rows are staged whole with their 16-byte units
  // permuted as the chain stages k rows, and read back in the same natural
  // map; rows past the sequence end repeat its last row (their outputs are
  // not stored, and each output column depends only on its own q row).
  const float fqv = p.scal[((int64_t)c * p.Hv + h) * (kScalars * kChunk) + 2 * kChunk + (tid & 63)];
  {
    constexpr int kVec = 16 / (int)sizeof(T);
    constexpr int kRowUnits = kHeadDim / kVec;
    constexpr int kQCopies = kChunk * kRowUnits / 64;             // 1 KB each
    constexpr int kFragCopies = kFragElems / kVec / 64;
    const char* qb = reinterpret_cast<const char*>(p.q + (t0 * p.Hk + kh) * kHeadDim);
    const int64_t rs = (int64_t)p.Hk * kHeadDim * sizeof(T);
#pragma unroll
    for (int i = w; i < kQCopies; i += 4) {
      const int P = 64 * i + lane, row = P / kRowUnits, pos = P % kRowUnits;
      dma16(qb + min(row, L - 1) * rs + (pos ^ kswz(row)) * 16, sm.Q + 64 * i * kVec);
    }
    const T* mp = p.mp + ((int64_t)c * p.Hv + h) * (kTbFrags * kFragElems);
#pragma unroll
    for (int i = w; i < kTbFrags * kFragCopies; i += 4)
      if (!zero_frag_index(i / kFragCopies))
        dma16(mp + (64 * i + lane) * kVec, sm.MP + 64 * i * kVec);
  }
  // z of this lane's outputs (token 16tt + m, columns 32w + 16b + 4g..+3,
  // one 4-element load each, kept in the input format)
  using Z4 = typename std::conditional<sizeof(T) == 2, uint2, uint4>::type;
  Z4 zr[4][2];
  if (p.z) {
    const T* zb = p.z + t0 * (int64_t)p.Hv * kHeadDim + (int64_t)h * kHeadDim + 32 * w + 4 * g;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = min(16 * tt + m, L - 1);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        zr[tt][b] = *reinterpret_cast<const Z4*>(zb + (int64_t)tok * p.Hv * kHeadDim + 16 * b);
    }
  }
  // this wave's exported fragments (value-column blocks 2w, 2w+1)
  Frag<T> ha[2][4], va[2][2];
  {
    const int64_t fo = ((int64_t)c * p.Hv + h) * kDvBlocks + 2 * w;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        ha[b][kb] = load_packed(p.hc + ((fo + b) * 4 + kb) * kFragElems + lane * 8);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        va[b][kb] = load_packed(p.vp + ((fo + b) * 2 + kb) * kFragElems + lane * 8);
    }
  }
  if (tid < kChunk) sm.fq[tid] = fqv;
  // the copies land in LDS: wait for them (and so for every load above)
  // before the barrier makes them visible
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));  // vmcnt(0)
  __syncthreads();

  // acc[b][tt]: lane (g, n) holds O[16tt + n][32w + 16b + 4g + rr]
  f32x4 acc[2][4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    Frag<T> qb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      qb[kb] = k_frag<T>(sm.Q, tt, kb, lane);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      acc[b][tt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(acc[b][tt], ha[b][kb], qb[kb]);
    }
  }
  // the columns of O^T are tokens: scale by fq of token 16tt + m
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const float f = sm.fq[scal_index(16 * tt + m)];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[b][tt][rr] *= f;
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    Frag<T> mb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (!zero_frag_index(2 * tt + kb))
        mb[kb] = *reinterpret_cast<const Frag<T>*>(&sm.MP[((2 * tt + kb) * 64 + lane) * 8]);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (!zero_frag_index(2 * tt + kb)) mma(acc[b][tt], va[b][kb], mb[kb]);
  }

  const int64_t vstride = (int64_t)p.Hv * kHeadDim;
  T* obase = p.o + t0 * vstride + (int64_t)h * kHeadDim + 32 * w + 4 * g;
  if (p.z) {
    // (z was loaded at the start: zr[tt][b][rr])
    // row sums of squares: this lane's 8 values, then lane groups, then waves
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float x = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x += acc[b][tt][rr] * acc[b][tt][rr];
      x = half_pair_sum(row_pair_sum(x));  // the lane groups (rows)
      if (g == 0) sm.ss[w][16 * tt + m] = x;
    }
    __syncthreads();
    float wv[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) wv[b][rr] = p.norm_w[32 * w + 16 * b + 4 * g + rr];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = 16 * tt + m;
      if (tok >= L) continue;
      const float tot = sm.ss[0][tok] + sm.ss[1][tok] + sm.ss[2][tok] + sm.ss[3][tok];
      const float rinv = rsqrt_fast(tot * (1.f / kHeadDim) + p.norm_eps);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float y[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float zf = z_elem<T>(zr[tt][b], rr);
          y[rr] = acc[b][tt][rr] * rinv * wv[b][rr] * silu_fast(zf);
        }
        store4(obase + tok * vstride + 16 * b, y);
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = 16 * tt + m;
      if (tok >= L) continue;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float y[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) y[rr] = acc[b][tt][rr];
        store4(obase + tok * vstride + 16 * b, y);
      }
    }
  }
}

// ------------------------------------------------------------- launches ----

// The prep and chain kernels use more LDS than the 64 KB default: raise the
// limit once per device and kernel.
static hipError_t allow_lds(const void* fn, size_t bytes,
                            unsigned long long* mask) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const unsigned long long bit = 1ull << (dev & 63);
  if (__atomic_load_n(mask, __ATOMIC_ACQUIRE) & bit) return hipSuccess;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes);
  if (err == hipSuccess) __atomic_fetch_or(mask, bit, __ATOMIC_RELEASE);
  return err;
}

template <typename T>
static hipError_t launch_typed(const PrefillLaunch& p, hipStream_t st,
                               hipEvent_t* ev, unsigned* ran) {
  hipError_t err;
  // Timing events (measurement only): stage i's pair is attached to its
  // kernel's dispatch, so it brackets that kernel's execution alone; a
  // stage with nothing to launch records nothing and is marked as not run.
  auto t0 = [&](int i) -> hipEvent_t { return ev ? ev[2 * i] : nullptr; };
  auto t1 = [&](int i) -> hipEvent_t { return ev ? ev[2 * i + 1] : nullptr; };
  auto empty = [&](int i) -> hipError_t {
    if (ran) *ran &= ~(1u << i);
    return hipSuccess;
  };
  T* tb = reinterpret_cast<T*>(p.ws + p.lay.tb);
  T* mp = reinterpret_cast<T*>(p.ws + p.lay.mp);
  float* scal = reinterpret_cast<float*>(p.ws + p.lay.scal);
  T* hc = reinterpret_cast<T*>(p.ws + p.lay.hc);
  T* vp = reinterpret_cast<T*>(p.ws + p.lay.vp);
  const int r = p.Hv / p.Hk;

  if (p.T == 0 && (err = empty(0)) != hipSuccess) return err;
  if (p.T > 0) {
    const size_t smem = sizeof(PrepSmem<T>);
    PrepArgs<T> a;
    a.q = static_cast<const T*>(p.q);
    a.k = static_cast<const T*>(p.k);
    a.a = static_cast<const T*>(p.a);
    a.b = static_cast<const T*>(p.b);
    a.A_log = p.A_log;
    a.dt_bias = p.dt_bias;
    a.N = p.N;
    a.Hk = p.Hk;
    a.Hv = p.Hv;
    a.r = r;
    a.T_tot = p.T;
    a.scale = p.scale;
    a.l2_eps = p.l2_eps;
    a.cu = p.cu_seqlens;
    a.tb = tb;
    a.mp = mp;
    a.scal = scal;
    a.slots = p.lay.max_chunks;
    a.cv = p.conv ? *p.conv : PrepConv{};
    a.qo = static_cast<T*>(const_cast<void*>(p.q));
    a.ko = static_cast<T*>(const_cast<void*>(p.k));
    a.vo = static_cast<T*>(const_cast<void*>(p.v));
    const dim3 grid(slot_head_blocks(p.lay.max_chunks, p.Hk, r));
    // the prep variant: plain, or with the layer's conv of width 1..4 (bf16)
    auto launch_prep = [&](auto kernel, unsigned long long* mask) -> hipError_t {
      hipError_t e = allow_lds((const void*)kernel, smem, mask);
      if (e != hipSuccess) return e;
      hipExtLaunchKernelGGL(kernel, grid, dim3(256), (uint32_t)smem, st, t0(0), t1(0), 0, a);
      return hipGetLastError();
    };
    static unsigned long long masks[5] = {0ull, 0ull, 0ull, 0ull, 0ull};
    if constexpr (sizeof(T) == 2) {
      switch (p.conv ? p.conv->W : 0) {
        case 1: err = launch_prep(prep_kernel<T, 1>, &masks[1]); break;
        case 2: err = launch_prep(prep_kernel<T, 2>, &masks[2]); break;
        case 3: err = launch_prep(prep_kernel<T, 3>, &masks[3]); break;
        case 4: err = launch_prep(prep_kernel<T, 4>, &masks[4]); break;
        default: err = launch_prep(prep_kernel<T, 0>, &masks[0]); break;
      }
    } else {
      err = launch_prep(prep_kernel<T, 0>, &masks[0]);
    }
    if (err != hipSuccess) return err;
  }

  {
    ChainArgs<T> a;
    a.k = static_cast<const T*>(p.k);
    a.v = static_cast<const T*>(p.v);
    a.state_in = p.state_in;
    a.state_out = p.state_out;
    a.N = p.N;
    a.Hk = p.Hk;
    a.Hv = p.Hv;
    a.r = r;
    a.T_tot = p.T;
    a.cu = p.cu_seqlens;
    a.tb = tb;
    a.scal = scal;
    a.hc = hc;
    a.vp = vp;
    a.seg_mode = 0;
    a.seg_chunks = 0;
    a.nseg = 0;
    a.seg_S = a.seg_B = a.seg_M = nullptr;
    const int64_t units = (int64_t)p.N * p.Hv;
    const int64_t units8 = (units + 7) / 8 * 8;
    // bf16 with more blocks than CUs: two slots, so that two blocks share
    // each CU; otherwise (fp32, or one block per CU) the deeper ring
    auto launch_chain = [&](dim3 grid, int64_t real_blocks, hipEvent_t e0,
                            hipEvent_t e1) -> hipError_t {
      hipError_t e;
      if (sizeof(T) == 2 && real_blocks > 2 * kChainCUs && p.T <= kChunk * (int64_t)p.N) {
        // many short sequences (one chunk each on average), more blocks
        // than one round at two per CU: one slot (35 KB), four blocks per
        // CU
        static unsigned long long mask1 = 0ull;
        const size_t smem = sizeof(ChainSmem<T, 1>);
        if ((e = allow_lds((const void*)chain_kernel<T, 1>, smem, &mask1)) != hipSuccess)
          return e;
        hipExtLaunchKernelGGL(chain_kernel<T, 1>, grid, dim3(320), (uint32_t)smem, st, e0, e1,
                              0, a);
      } else if (sizeof(T) == 2 && real_blocks > kChainCUs) {
        static unsigned long long mask2 = 0ull;
        const size_t smem = sizeof(ChainSmem<T, 2>);
        if ((e = allow_lds((const void*)chain_kernel<T, 2>, smem, &mask2)) != hipSuccess)
          return e;
        hipExtLaunchKernelGGL(chain_kernel<T, 2>, grid, dim3(320), (uint32_t)smem, st, e0, e1,
                              0, a);
      } else {
        constexpr int kDeep = sizeof(T) == 2 ? 4 : 2;
        static unsigned long long maskd = 0ull;
        const size_t smem = sizeof(ChainSmem<T, kDeep>);
        if ((e = allow_lds((const void*)chain_kernel<T, kDeep>, smem, &maskd)) != hipSuccess)
          return e;
        hipExtLaunchKernelGGL(chain_kernel<T, kDeep>, grid, dim3(320), (uint32_t)smem, st, e0,
                              e1, 0, a);
      }
      return hipGetLastError();
    };
    const unsigned gx = (unsigned)(units8 * kDvBlocks);
    const int G = p.scan_segments;
    if (G < 2) {
      if ((err = launch_chain(dim3(gx), units8 * kDvBlocks, t0(1), t1(1))) != hipSuccess)
        return err;
    } else {
      // the sequence-parallel scan of one sequence: pass A (segment 0 and
      // the segment maps), the start states in order, pass C (segments 1..)
      a.seg_chunks = p.seg_chunks;
      a.nseg = G;
      a.seg_S = reinterpret_cast<float*>(p.ws + p.lay.seg_S);
      a.seg_B = reinterpret_cast<float*>(p.ws + p.lay.seg_B);
      a.seg_M = reinterpret_cast<float*>(p.ws + p.lay.seg_M);
      a.seg_mode = 1;
      const int64_t runs_a = units * (2 * G - 3), runs_c = units * (G - 1);
      if ((err = launch_chain(dim3((unsigned)((runs_a + 7) / 8 * 8 * kDvBlocks)),
                              runs_a * kDvBlocks, t0(1), nullptr)) != hipSuccess)
        return err;
      if (G >= 3) {
        CombineArgs c;
        c.seg_S = a.seg_S;
        c.seg_B = a.seg_B;
        c.seg_M = a.seg_M;
        c.units = (int)units;
        c.nseg = G;
        static unsigned long long cmask = 0ull;
        if ((err = allow_lds((const void*)scan_combine_kernel, sizeof(CombineSmem), &cmask)) !=
            hipSuccess)
          return err;
        hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)units, kHeadDim / kCombineRows),
                           dim3(256),
                           (uint32_t)sizeof(CombineSmem), st, c);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      a.seg_mode = 2;
      if ((err = launch_chain(dim3((unsigned)((runs_c + 7) / 8 * 8 * kDvBlocks)),
                              runs_c * kDvBlocks, nullptr, t1(1))) != hipSuccess)
        return err;
    }
  }

  if (p.T > 0) {
    static unsigned long long out_mask = 0ull;
    const size_t smem = sizeof(OutSmem<T>);
    if ((err = allow_lds((const void*)out_kernel<T>, smem, &out_mask)) != hipSuccess)
      return err;
    OutArgs<T> a;
    a.q = static_cast<const T*>(p.q);
    a.z = static_cast<const T*>(p.z);
    a.norm_w = p.norm_w;
    a.o = static_cast<T*>(p.o);
    a.N = p.N;
    a.Hk = p.Hk;
    a.Hv = p.Hv;
    a.r = r;
    a.T_tot = p.T;
    a.norm_eps = p.norm_eps;
    a.cu = p.cu_seqlens;
    a.mp = mp;
    a.hc = hc;
    a.vp = vp;
    a.scal = scal;
    a.slots = p.lay.max_chunks;
    hipExtLaunchKernelGGL(out_kernel<T>, dim3(slot_head_blocks(p.lay.max_chunks, p.Hk, r)),
                          dim3(256), (uint32_t)smem, st, t0(2), t1(2), 0, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (p.T == 0 && (err = empty(2)) != hipSuccess) return err;
  return empty(kStageShort);
}

uint64_t prefill_grid_work_items(int64_t max_chunks, int64_t N, int Hk, int Hv,
                                 int scan_segments) {
  // prep and out: 256 threads per (chunk slot, value head) block
  const uint64_t slot_items = slot_head_blocks64(max_chunks, Hk, Hv / Hk) * 256;
  // chain: 320 threads per (run, 16-column block), runs padded to 8; the
  // scan's pass A runs each head 2G - 3 times
  const int64_t units = N * (int64_t)Hv;
  const int64_t runs = scan_segments >= 2 ? units * (2 * (int64_t)scan_segments - 3) : units;
  const uint64_t chain_items = (uint64_t)((runs + 7) / 8 * 8) * kDvBlocks * 320;
  return slot_items > chain_items ? slot_items : chain_items;
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream,
                          hipEvent_t* stage_events, unsigned* stage_ran) {
  if (p.dtype == 1) return launch_typed<__bf16>(p, stream, stage_events, stage_ran);
  return launch_typed<float>(p, stream, stage_events, stage_ran);
}

// ------------------------------------------------- no-allocation scratch ----
//
// The workspace of gdn_prefill_noalloc: a file-scope device array that each
// GPU the library runs on holds until the process ends.  In host code
// `scratch` names a host-side stand-in, not the device array: its device
// address is looked up once per device (with that device current) and kept,
// and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gdn
