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
//   plan  : sequence table and chunk prefix sums from cu_seqlens (1 block)
//   prep  : per (chunk, key head): norms, the two Gram products, and per
//           value head the gates, Tb and MP as packed MFMA fragments
//           (parallel over chunks)
//   chain : per (sequence, value head, 16-column block of the state): the
//           sequential pass over chunks, H in registers (fp32), operands
//           staged through LDS one chunk ahead, chunk outputs written as
//           they are produced
//   norm  : gated RMSNorm over each (token, value head) row, in place on o
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdn_frag.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// ---------------------------------------------------------------- plan ----

// Out-of-range cu_seqlens values are clamped into [0, T] and the chunk
// prefix sums are capped at max_chunks (the workspace's chunk capacity), so
// every later access stays inside the inputs and the workspace.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* cu, int N,
                                                    int64_t T,
                                                    int32_t max_chunks,
                                                    int32_t* seq_start,
                                                    int32_t* seq_len,
                                                    int32_t* chunk_start) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int nch = 0;
    if (n < N) {
      int64_t s = cu ? (int64_t)cu[n] : 0;
      int64_t e = cu ? (int64_t)cu[n + 1] : T;
      s = s < 0 ? 0 : (s > T ? T : s);
      e = e < s ? s : (e > T ? T : e);
      seq_start[n] = (int32_t)s;
      seq_len[n] = (int32_t)(e - s);
      nch = (int)((e - s + kChunk - 1) / kChunk);
    }
    int x = nch;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
      int y = lane < 16 ? wsum[lane] : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int z = __shfl_up(y, off);
        if (lane >= off) y += z;
      }
      if (lane < 16) wsum[lane] = y;
    }
    __syncthreads();
    const int incl = (w > 0 ? wsum[w - 1] : 0) + x;
    const int carry = carry_s;
    if (n < N) chunk_start[n + 1] = min(carry + incl, max_chunks);
    __syncthreads();
    if (tid == 1023) carry_s = carry + incl;
    __syncthreads();
  }
  if (tid == 0) chunk_start[0] = 0;
}

// ---------------------------------------------------------------- prep ----

template <typename T>
struct PrepArgs {
  const T *q, *k, *a, *b;
  const float *A_log, *dt_bias;
  int N, Hk, Hv, r;
  float scale, l2_eps;
  const int32_t *seq_start, *seq_len, *chunk_start;
  T *tb, *mp;
  float* scal;
};

template <typename T>
struct PrepSmem {
  static constexpr int kLd = 128 + 16 / (int)sizeof(T);  // row pad of 16 B
  union {
    struct {
      T Ks[kChunk][kLd];
      T Qs[kChunk][kLd];
    } in;  // raw rows, until the Gram products are done
    struct {
      float Am[kChunk][kChunk + 1];  // A (strictly lower)
      float Tm[kChunk][kChunk + 1];  // MP, then (I + A)^{-1}
    } inv;
  } u;
  float Gm[kChunk][kChunk + 1];  // raw K K^T (blocks on/below the diagonal)
  float Pm[kChunk][kChunk + 1];  // raw Q K^T (blocks on/below the diagonal)
  float Xm[4][16][17];           // per-wave block products
  float rk[kChunk], rq[kChunk], gam[kChunk], bet[kChunk];
};

// Sequence owning chunk c: the largest n with chunk_start[n] <= c.
__device__ __forceinline__ int find_seq(const int32_t* chunk_start, int N,
                                        int c) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_start[mid] <= c)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// acc += X[ra.., ca..] (16x16) * Y[rb.., cb..] (16x16), fp32 MFMA.
__device__ __forceinline__ void mma16_f32(f32x4& acc, const float (*X)[kChunk + 1],
                                          int ra, int ca,
                                          const float (*Y)[kChunk + 1], int rb,
                                          int cb, int m, int g) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[ra + m][ca + 4 * kk + g],
                                               Y[rb + 4 * kk + g][cb + m], acc,
                                               0, 0, 0);
}

template <typename T>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs<T> p) {
  extern __shared__ __align__(16) char smem_raw[];
  PrepSmem<T>& sm = *reinterpret_cast<PrepSmem<T>*>(smem_raw);
  const int c = blockIdx.x;
  const int kh = blockIdx.y;
  if (c >= p.chunk_start[p.N]) return;
  const int n = find_seq(p.chunk_start, p.N, c);
  const int jc = c - p.chunk_start[n];
  const int64_t t0 = (int64_t)p.seq_start[n] + (int64_t)jc * kChunk;
  const int L = min(kChunk, p.seq_len[n] - jc * kChunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m16 = lane & 15;

  // 1. the chunk's raw q and k rows (zero rows past the sequence end)
  {
    constexpr int kVec = 16 / sizeof(T);
    constexpr int kPieces = kHeadDim / kVec;
    constexpr int kRowsPerPass = 256 / kPieces;
    const int pc = tid % kPieces;
    for (int rr = tid / kPieces; rr < kChunk; rr += kRowsPerPass) {
      uint4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
      if (rr < L) {
        const int64_t off = ((t0 + rr) * p.Hk + kh) * kHeadDim + pc * kVec;
        kv = *reinterpret_cast<const uint4*>(p.k + off);
        qv = *reinterpret_cast<const uint4*>(p.q + off);
      }
      *reinterpret_cast<uint4*>(&sm.u.in.Ks[rr][pc * kVec]) = kv;
      *reinterpret_cast<uint4*>(&sm.u.in.Qs[rr][pc * kVec]) = qv;
    }
  }
  __syncthreads();

  // 2. inverse L2 norms (4 threads per row)
  {
    const int row = tid >> 2, part = tid & 3;
    float sk = 0.f, sq = 0.f;
#pragma unroll 8
    for (int e = 0; e < 32; ++e) {
      const float kx = to_f32(sm.u.in.Ks[row][part * 32 + e]);
      const float qx = to_f32(sm.u.in.Qs[row][part * 32 + e]);
      sk += kx * kx;
      sq += qx * qx;
    }
    sk += __shfl_xor(sk, 1);
    sk += __shfl_xor(sk, 2);
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    if (part == 0) {
      sm.rk[row] = 1.f / sqrtf(sk + p.l2_eps);
      sm.rq[row] = p.scale / sqrtf(sq + p.l2_eps);
    }
  }

  // 3. raw Gram tiles on and below the diagonal: G = K K^T, P = Q K^T
  for (int job = wave; job < 20; job += 4) {
    const int which = job / 10;
    const int jj = job % 10;
    const int i = (jj >= 6) ? 3 : (jj >= 3) ? 2 : (jj >= 1) ? 1 : 0;
    const int j = jj - i * (i + 1) / 2;
    const T* xrow = which ? &sm.u.in.Qs[16 * i + m16][0] : &sm.u.in.Ks[16 * i + m16][0];
    const T* krow = &sm.u.in.Ks[16 * j + m16][0];
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      mma(acc, load_frag(xrow + 32 * kb, g), load_frag(krow + 32 * kb, g));
    float(*D)[kChunk + 1] = which ? sm.Pm : sm.Gm;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) D[16 * i + 4 * g + rr][16 * j + m16] = acc[rr];
  }
  __syncthreads();  // q/k rows are dead from here; Am/Tm reuse their space

  // 4. per value head of this key head
  for (int u = 0; u < p.r; ++u) {
    const int h = kh * p.r + u;
    float* sc = p.scal + ((int64_t)c * p.Hv + h) * (kScalars * kChunk);
    if (wave == 0) {
      const int t = lane;
      float gg = 0.f, bb = 0.f;
      if (t < L) {
        const int64_t idx = (t0 + t) * p.Hv + h;
        const float x = to_f32(p.a[idx]) + p.dt_bias[h];
        const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
        gg = -expf(p.A_log[h]) * sp;
        bb = 1.f / (1.f + expf(-to_f32(p.b[idx])));
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(gg, off);
        if (lane >= off) gg += y;
      }
      sm.gam[t] = gg;
      sm.bet[t] = bb;
      const float gL = __shfl(gg, 63);
      const float eg = expf(gg);
      sc[t] = eg * sm.rk[t];
      sc[kChunk + t] = expf(gL - gg) * sm.rk[t];
      sc[2 * kChunk + t] = eg * sm.rq[t];
      sc[3 * kChunk + t] = expf(gL);
    }
    __syncthreads();

    // A (strictly lower) and MP (lower incl. diagonal, staged in Tm); the
    // decay e^{gamma_t - gamma_s} is formed once per (t >= s)
    for (int e = tid; e < kChunk * kChunk; e += 256) {
      const int t = e >> 6, s = e & 63;
      float av = 0.f, mv = 0.f;
      if (t >= s) {
        const float dec = expf(sm.gam[t] - sm.gam[s]);
        mv = dec * sm.Pm[t][s] * sm.rq[t] * sm.rk[s];
        if (t > s) av = sm.bet[t] * dec * sm.Gm[t][s] * sm.rk[t] * sm.rk[s];
      }
      sm.u.inv.Am[t][s] = av;
      sm.u.inv.Tm[t][s] = mv;
    }
    __syncthreads();
    {
      T* dst = p.mp + ((int64_t)c * p.Hv + h) * (kTbFrags * kFragElems);
      for (int pr = tid; pr < kTbFrags * 64; pr += 256) {
        const int f = pr >> 6, l = pr & 63;
        const int i = f >> 1, kb = f & 1;
        const int t = 16 * i + (l & 15), gg = l >> 4;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = sm.u.inv.Tm[t][32 * kb + kperm(gg, j)];
        store_packed(dst + f * kFragElems + l * 8, x);
      }
    }
    __syncthreads();

    // (I + A)^{-1}: diagonal 16x16 blocks by forward substitution (wave w
    // owns block w, lane = column); upper parts of the blocks get 0 ...
    if (lane < 16) {
      const int bi = wave, cc = lane;
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float acc = (rr == cc) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < rr; ++s) acc -= sm.u.inv.Am[16 * bi + rr][16 * bi + s] * x[s];
        x[rr] = acc;
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.u.inv.Tm[16 * bi + rr][16 * bi + cc] = x[rr];
    }
    // ... and everything above the diagonal blocks is 0
    for (int e = tid; e < kChunk * kChunk; e += 256) {
      const int t = e >> 6, s = e & 63;
      if ((s >> 4) > (t >> 4)) sm.u.inv.Tm[t][s] = 0.f;
    }
    __syncthreads();
    // ... then block (i, j), i > j, by distance d = i - j:
    //     T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj     (fp32 MFMA, one wave
    //     per block; the blocks of one distance are independent)
    for (int d = 1; d < 4; ++d) {
      if (wave < 4 - d) {
        const int j = wave, i = j + d;
        f32x4 x = zero4();
        for (int kk = j; kk < i; ++kk)
          mma16_f32(x, sm.u.inv.Am, 16 * i, 16 * kk, sm.u.inv.Tm, 16 * kk, 16 * j,
                    m16, g);
        float(*X)[17] = sm.Xm[wave];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) X[4 * g + rr][m16] = x[rr];
        // other lanes of this wave read X next: order the LDS accesses
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 y = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(
              sm.u.inv.Tm[16 * i + m16][16 * i + 4 * kk + g], X[4 * kk + g][m16], y,
              0, 0, 0);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sm.u.inv.Tm[16 * i + 4 * g + rr][16 * j + m16] = -y[rr];
      }
      __syncthreads();
    }

    // Tb = T diag(beta) as A-operand fragments [token t][token s]
    {
      T* dst = p.tb + ((int64_t)c * p.Hv + h) * (kTbFrags * kFragElems);
      for (int pr = tid; pr < kTbFrags * 64; pr += 256) {
        const int f = pr >> 6, l = pr & 63;
        const int i = f >> 1, kb = f & 1;
        const int t = 16 * i + (l & 15), gg = l >> 4;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int s = 32 * kb + kperm(gg, j);
          x[j] = sm.u.inv.Tm[t][s] * sm.bet[s];
        }
        store_packed(dst + f * kFragElems + l * 8, x);
      }
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------- chain ----

template <typename T>
struct ChainArgs {
  const T *q, *k, *v;
  const float* state_in;
  float* state_out;
  T* o;
  int N, Hk, Hv, r;
  const int32_t *seq_start, *seq_len, *chunk_start;
  const T *tb, *mp;
  const float* scal;
};

// One chunk's operands as the chain block stages them in LDS.
template <typename T>
struct ChainStage {
  static constexpr int kLd = 128 + 16 / (int)sizeof(T);
  T Ks[kChunk][kLd];                 // raw k rows
  T Qs[kChunk][kLd];                 // raw q rows
  T Tbf[kTbFrags * kFragElems];      // packed Tb fragments
  T MPf[kTbFrags * kFragElems];      // packed MP fragments
  T Vs[kChunk][kDvBlock];            // this block's 16 value columns
  float Sc[kScalars * kChunk];       // ek, fk, fq, e^{gamma_L}
};

template <typename T>
struct ChainSmem {
  static constexpr int kStages = sizeof(T) == 2 ? 2 : 1;
  ChainStage<T> st[kStages];
  T Hx[4 * kFragElems];  // H (bf16/fp32) as the 4 B-operand k-groups over dk
  T Rx[2 * kFragElems];  // R as B operand over tokens
  T Vx[2 * kFragElems];  // V' as B operand over tokens
  T Wx[2 * kFragElems];  // diag(fk) V' as B operand over tokens
};

// Global -> register staging of one chunk (all 256 threads), then register
// -> LDS.  16-byte pieces; rows past the sequence end are zero.
template <typename T>
struct StageRegs {
  static constexpr int kRowPieces = kHeadDim * (int)sizeof(T) / 16;  // per row
  static constexpr int kQK = kChunk * kRowPieces / 256;             // per thread
  static constexpr int kFr = kTbFrags * kFragElems * (int)sizeof(T) / 16 / 256;
  static constexpr int kVPieces = kChunk * kDvBlock * (int)sizeof(T) / 16;
  uint4 k[kQK], q[kQK], tb[kFr], mp[kFr], v, sc;
};

template <typename T>
__device__ __forceinline__ void stage_load(StageRegs<T>& R, const ChainArgs<T>& p,
                                           int c, int64_t t0, int L, int h,
                                           int kh, int dvb, int tid) {
  using S = StageRegs<T>;
  constexpr int kVec = 16 / sizeof(T);
#pragma unroll
  for (int i = 0; i < S::kQK; ++i) {
    const int pc = tid + 256 * i;
    const int row = pc / S::kRowPieces, col = (pc % S::kRowPieces) * kVec;
    uint4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
    if (row < L) {
      const int64_t off = ((t0 + row) * p.Hk + kh) * kHeadDim + col;
      kv = *reinterpret_cast<const uint4*>(p.k + off);
      qv = *reinterpret_cast<const uint4*>(p.q + off);
    }
    R.k[i] = kv;
    R.q[i] = qv;
  }
  const int64_t fbase = ((int64_t)c * p.Hv + h) * (kTbFrags * kFragElems);
#pragma unroll
  for (int i = 0; i < S::kFr; ++i) {
    R.tb[i] = reinterpret_cast<const uint4*>(p.tb + fbase)[tid + 256 * i];
    R.mp[i] = reinterpret_cast<const uint4*>(p.mp + fbase)[tid + 256 * i];
  }
  R.v = uint4{0u, 0u, 0u, 0u};
  if (tid < S::kVPieces) {
    constexpr int kPerRow = kDvBlock / kVec;
    const int row = tid / kPerRow, col = (tid % kPerRow) * kVec;
    if (row < L)
      R.v = *reinterpret_cast<const uint4*>(
          p.v + ((t0 + row) * p.Hv + h) * kHeadDim + dvb * kDvBlock + col);
  }
  R.sc = uint4{0u, 0u, 0u, 0u};
  if (tid < kScalars * kChunk / 4)
    R.sc = reinterpret_cast<const uint4*>(
        p.scal + ((int64_t)c * p.Hv + h) * (kScalars * kChunk))[tid];
}

template <typename T>
__device__ __forceinline__ void stage_store(const StageRegs<T>& R,
                                            ChainStage<T>& st, int tid) {
  using S = StageRegs<T>;
  constexpr int kVec = 16 / sizeof(T);
#pragma unroll
  for (int i = 0; i < S::kQK; ++i) {
    const int pc = tid + 256 * i;
    const int row = pc / S::kRowPieces, col = (pc % S::kRowPieces) * kVec;
    *reinterpret_cast<uint4*>(&st.Ks[row][col]) = R.k[i];
    *reinterpret_cast<uint4*>(&st.Qs[row][col]) = R.q[i];
  }
#pragma unroll
  for (int i = 0; i < S::kFr; ++i) {
    reinterpret_cast<uint4*>(st.Tbf)[tid + 256 * i] = R.tb[i];
    reinterpret_cast<uint4*>(st.MPf)[tid + 256 * i] = R.mp[i];
  }
  if (tid < S::kVPieces) {
    constexpr int kPerRow = kDvBlock / kVec;
    const int row = tid / kPerRow, col = (tid % kPerRow) * kVec;
    *reinterpret_cast<uint4*>(&st.Vs[row][col]) = R.v;
  }
  if (tid < kScalars * kChunk / 4) reinterpret_cast<uint4*>(st.Sc)[tid] = R.sc;
}

// Writes the 4 values of one 16-row accumulator tile into its half of a
// B-operand fragment buffer (k-group = tile / 2, half = tile % 2).
template <typename T>
__device__ __forceinline__ void put_half(T* buf, int tile, int lane,
                                         const float (&x)[4]) {
  T* dst = buf + (tile >> 1) * kFragElems + lane * 8 + 4 * (tile & 1);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) dst[rr] = from_f32<T>(x[rr]);
}

// One block (4 waves) owns 16 value columns of one (sequence, value head)
// state.  Wave w owns token tile w (rows 16w..16w+15) of every per-chunk
// product and dk rows 32w..32w+31 of the state; the waves exchange R, V' and
// H through LDS, three barriers per chunk.  The next chunk's operands are
// loaded into registers while the current one is computed and written to the
// other LDS stage at its end.  Block ids put the 8 column blocks of a head
// on one XCD (same blockIdx % 8), so they share that XCD's L2.
template <typename T>
__global__ __launch_bounds__(256) void chain_kernel(ChainArgs<T> p) {
  extern __shared__ __align__(16) char smem_raw[];
  ChainSmem<T>& sm = *reinterpret_cast<ChainSmem<T>*>(smem_raw);
  constexpr int kStages = ChainSmem<T>::kStages;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, s8 = bid >> 3;
  const int unit = (s8 >> 3) * 8 + xcd;
  const int dvb = s8 & 7;
  if (unit >= p.N * p.Hv) return;
  const int n = unit / p.Hv, h = unit % p.Hv, kh = h / p.r;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, m16 = lane & 15;
  const int dv = dvb * kDvBlock + m16;

  // state rows dk = 32w + 16t + 4g + rr, column dv
  f32x4 H[2];
  const size_t sbase = ((size_t)unit * kHeadDim + dv) * kHeadDim;
#pragma unroll
  for (int t = 0; t < 2; ++t)
    H[t] = p.state_in ? *reinterpret_cast<const f32x4*>(p.state_in + sbase +
                                                        32 * w + 16 * t + 4 * g)
                      : zero4();
  {
    const Frag<T> f = frag_from_acc_t<T>(H[0], H[1]);
    *reinterpret_cast<Frag<T>*>(&sm.Hx[w * kFragElems + lane * 8]) = f;
  }

  const int c_begin = p.chunk_start[n], c_end = p.chunk_start[n + 1];
  const int64_t seq0 = p.seq_start[n];
  const int len = p.seq_len[n];
  const int64_t vstride = (int64_t)p.Hv * kHeadDim;

  StageRegs<T> R;
  if (c_begin < c_end) {
    stage_load(R, p, c_begin, seq0, min(kChunk, len), h, kh, dvb, tid);
    stage_store(R, sm.st[0], tid);
  }
  __syncthreads();

  for (int c = c_begin; c < c_end; ++c) {
    const int jc = c - c_begin;
    const int64_t t0 = seq0 + (int64_t)jc * kChunk;
    const int L = min(kChunk, len - jc * kChunk);
    const int si = kStages == 2 ? (jc & 1) : 0;
    ChainStage<T>& S = sm.st[si];
    const bool more = c + 1 < c_end;
    if (kStages == 2 && more)
      stage_load(R, p, c + 1, t0 + kChunk, min(kChunk, len - (jc + 1) * kChunk), h,
                 kh, dvb, tid);

    // 1. Y = K H and Q H for token tile w (H = state at chunk entry)
    Frag<T> hb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      hb[kb] = *reinterpret_cast<const Frag<T>*>(&sm.Hx[kb * kFragElems + lane * 8]);
    f32x4 Y = zero4(), O = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      mma(Y, load_frag(&S.Ks[16 * w + m16][32 * kb], g), hb[kb]);
      mma(O, load_frag(&S.Qs[16 * w + m16][32 * kb], g), hb[kb]);
    }
    // 2. R = V - diag(e^gamma rk) Y
    {
      const f32x4 ek = *reinterpret_cast<const f32x4*>(&S.Sc[16 * w + 4 * g]);
      float r[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        r[rr] = to_f32(S.Vs[16 * w + 4 * g + rr][m16]) - ek[rr] * Y[rr];
      put_half(sm.Rx, w, lane, r);
    }
    __syncthreads();
    // 3. V' = Tb R for token tile w
    f32x4 Vp = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      mma(Vp, *reinterpret_cast<const Frag<T>*>(&S.Tbf[(2 * w + kb) * kFragElems + lane * 8]),
          *reinterpret_cast<const Frag<T>*>(&sm.Rx[kb * kFragElems + lane * 8]));
    {
      const f32x4 fk = *reinterpret_cast<const f32x4*>(&S.Sc[kChunk + 16 * w + 4 * g]);
      float vv[4], ww[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        vv[rr] = Vp[rr];
        ww[rr] = Vp[rr] * fk[rr];
      }
      put_half(sm.Vx, w, lane, vv);
      put_half(sm.Wx, w, lane, ww);
    }
    __syncthreads();
    // 4. O = diag(e^gamma rq) Q H + MP V' for token tile w
    {
      const f32x4 fq = *reinterpret_cast<const f32x4*>(&S.Sc[2 * kChunk + 16 * w + 4 * g]);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) O[rr] *= fq[rr];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mma(O, *reinterpret_cast<const Frag<T>*>(&S.MPf[(2 * w + kb) * kFragElems + lane * 8]),
            *reinterpret_cast<const Frag<T>*>(&sm.Vx[kb * kFragElems + lane * 8]));
      T* obase = p.o + t0 * vstride + (int64_t)h * kHeadDim + dv;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tok = 16 * w + 4 * g + rr;
        if (tok < L) obase[tok * vstride] = from_f32<T>(O[rr]);
      }
    }
    // 5. H <- e^{gamma_L} H + K^T diag(fk) V' for dk rows 32w..32w+31; the
    //    K^T operand is read transposed from the staged k rows
    {
      const float eL = S.Sc[3 * kChunk];
      Frag<T> wb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        wb[kb] = *reinterpret_cast<const Frag<T>*>(&sm.Wx[kb * kFragElems + lane * 8]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) H[t][rr] *= eL;
        const int dk = 32 * w + 16 * t + m16;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          Frag<T> a;
#pragma unroll
          for (int j = 0; j < 8; ++j) a.v[j] = S.Ks[32 * kb + kperm(g, j)][dk];
          mma(H[t], a, wb[kb]);
        }
      }
      const Frag<T> f = frag_from_acc_t<T>(H[0], H[1]);
      *reinterpret_cast<Frag<T>*>(&sm.Hx[w * kFragElems + lane * 8]) = f;
    }
    if (kStages == 2 && more) stage_store(R, sm.st[si ^ 1], tid);
    __syncthreads();
    if (kStages == 1 && more) {
      stage_load(R, p, c + 1, t0 + kChunk, min(kChunk, len - (jc + 1) * kChunk), h,
                 kh, dvb, tid);
      stage_store(R, sm.st[0], tid);
      __syncthreads();
    }
  }

  if (p.state_out) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      *reinterpret_cast<f32x4*>(p.state_out + sbase + 32 * w + 16 * t + 4 * g) = H[t];
  }
}

// ---------------------------------------------------------------- norm ----

// y = o / sqrt(mean(o^2) + eps) * w * silu(z) over each 128-wide row; 16
// threads per row, 8 consecutive elements (one 16/32-byte access) each.
template <typename T>
__global__ __launch_bounds__(256) void norm_kernel(T* o, const T* z,
                                                   const float* w, int64_t rows,
                                                   float eps) {
  const int tid = threadIdx.x, sub = tid & 15;
  float wv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wv[j] = w[8 * sub + j];
  const int64_t stride = (int64_t)gridDim.x * 16;
  for (int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4); row < rows;
       row += stride) {
    T* op = o + row * kHeadDim + 8 * sub;
    const T* zp = z + row * kHeadDim + 8 * sub;
    float ov[8], zv[8];
    if constexpr (sizeof(T) == 2) {
      const Frag<T> a = load_packed(op);
      const Frag<T> b = load_packed(zp);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ov[j] = to_f32(a.v[j]);
        zv[j] = to_f32(b.v[j]);
      }
    } else {
      const Frag<T> a = load_packed(op);
      const Frag<T> b = load_packed(zp);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ov[j] = a.v[j];
        zv[j] = b.v[j];
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += ov[j] * ov[j];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off);
    const float rinv = 1.f / sqrtf(ss * (1.f / kHeadDim) + eps);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      y[j] = ov[j] * rinv * wv[j] * (zv[j] / (1.f + expf(-zv[j])));
    store_packed(op, y);
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
                               hipEvent_t* ev) {
  hipError_t err;
  auto rec = [&](int i) -> hipError_t {
    return ev ? hipEventRecord(ev[i], st) : hipSuccess;
  };
  int32_t* seq_start = reinterpret_cast<int32_t*>(p.ws + p.lay.seq_start);
  int32_t* seq_len = reinterpret_cast<int32_t*>(p.ws + p.lay.seq_len);
  int32_t* chunk_start = reinterpret_cast<int32_t*>(p.ws + p.lay.chunk_start);
  T* tb = reinterpret_cast<T*>(p.ws + p.lay.tb);
  T* mp = reinterpret_cast<T*>(p.ws + p.lay.mp);
  float* scal = reinterpret_cast<float*>(p.ws + p.lay.scal);
  const int r = p.Hv / p.Hk;

  if ((err = rec(0)) != hipSuccess) return err;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, p.cu_seqlens,
                     p.N, p.T, (int32_t)p.lay.max_chunks, seq_start, seq_len,
                     chunk_start);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = rec(1)) != hipSuccess) return err;

  if (p.T > 0) {
    static unsigned long long prep_mask = 0ull;
    const size_t smem = sizeof(PrepSmem<T>);
    if ((err = allow_lds((const void*)prep_kernel<T>, smem, &prep_mask)) !=
        hipSuccess)
      return err;
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
    a.scale = p.scale;
    a.l2_eps = p.l2_eps;
    a.seq_start = seq_start;
    a.seq_len = seq_len;
    a.chunk_start = chunk_start;
    a.tb = tb;
    a.mp = mp;
    a.scal = scal;
    hipLaunchKernelGGL(prep_kernel<T>, dim3((unsigned)p.lay.max_chunks, p.Hk),
                       dim3(256), smem, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = rec(2)) != hipSuccess) return err;

  {
    static unsigned long long chain_mask = 0ull;
    const size_t smem = sizeof(ChainSmem<T>);
    if ((err = allow_lds((const void*)chain_kernel<T>, smem, &chain_mask)) !=
        hipSuccess)
      return err;
    ChainArgs<T> a;
    a.q = static_cast<const T*>(p.q);
    a.k = static_cast<const T*>(p.k);
    a.v = static_cast<const T*>(p.v);
    a.state_in = p.state_in;
    a.state_out = p.state_out;
    a.o = static_cast<T*>(p.o);
    a.N = p.N;
    a.Hk = p.Hk;
    a.Hv = p.Hv;
    a.r = r;
    a.seq_start = seq_start;
    a.seq_len = seq_len;
    a.chunk_start = chunk_start;
    a.tb = tb;
    a.mp = mp;
    a.scal = scal;
    const int64_t units = (int64_t)p.N * p.Hv;
    const int64_t units8 = (units + 7) / 8 * 8;
    hipLaunchKernelGGL(chain_kernel<T>, dim3((unsigned)(units8 * kDvBlocks)),
                       dim3(256), smem, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = rec(3)) != hipSuccess) return err;

  if (p.z && p.T > 0) {
    const int64_t rows = p.T * p.Hv;
    int64_t blocks = (rows + 15) / 16;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(norm_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<T*>(p.o), static_cast<const T*>(p.z),
                       p.norm_w, rows, p.norm_eps);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return rec(4);
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream,
                          hipEvent_t* stage_events) {
  if (p.dtype == 1) return launch_typed<__bf16>(p, stream, stage_events);
  return launch_typed<float>(p, stream, stage_events);
}

}  // namespace gdn
