// gdn_layer.hip -- gfx950 kernels of the full Gated DeltaNet layer around
// the prefill: the bf16 projection GEMM and the depthwise causal conv1d +
// SiLU.
//
// Layer (the four input projections run as one GEMM, per "Add opt-in fused
// Qwen3.5 inference kernels" (JevAny PR #29), Summary; its packed output
// width 12,352 at the 4B geometry per "[Perf] Pack the Qwen3.5 GDN input
// projection on CUDA, including from the dense wrapper" (sglang PR #42126),
// Modifications):
//   P = x W_in^T                  columns q | k | v | z | b | a
//   q, k, v = silu(causal depthwise conv(P[:, q|k|v]))
//   y = gated delta rule prefill (q, k, v, a, b, z)   (gdn_prefill)
//   out = y W_out^T
// Weights are in the [out_features, in_features] layout, so both GEMM
// operands are contiguous along the contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_frag.hpp"
#include "gdn_internal.hpp"
#include "gdn_layer.hpp"
#include "gdn_math.hpp"

namespace gdn {

// ------------------------------------------------------------------ GEMM ----
//
// C[M][N] = A[M][K] * B[N][K]^T: bf16 operands, fp32 accumulation, bf16
// result.  Two kernels: gemm8_kernel (eight waves, two per SIMD, below) for
// K a multiple of 64, which covers the layer's projections, and
// gemm_kernel for the rest.  In gemm_kernel one block (four waves, 2 x 2)
// computes a BM x BN tile; wave (wr, wc) owns rows wr*BM/2.. and columns
// wc*BN/2.. of it.  The
// contraction runs in k-tiles of GK staged through a ring of ST LDS slots
// by direct global -> LDS copies, ST - 1 tiles ahead.  A staged operand
// keeps each row's GK * 2 bytes whole with its 16-byte units permuted
// (position pos of row r holds unit pos ^ swz(r)), so the fragment reads
// (16 rows x one unit per lane group) are free of bank conflicts.  With
// GK = 64 a row of a tile is one whole 128-byte line, so each copy fetches
// full lines.  Rows past M or N are read from the last valid row (every
// copy stays in bounds) and their results are not stored.
//
// The result's columns may go to up to four destinations: segment s covers
// columns [col0[s], col0[s + 1]) (the last one up to N) and stores column c
// of row r at ptr[s] + r * ld[s] + (c - col0[s]).  Segment starts may be
// any columns; the 16-byte stores below are used only when every start is
// a multiple of 8 (no 8-column piece then spans two segments).

template <int BM, int BN, int GK, int ST>
struct GemmSmem {
  __bf16 A[ST][BM * GK];
  __bf16 B[ST][BN * GK];
};

// Unit permutation of a staged row: 64-byte rows (GK = 32) use
// (row >> 2) & 3, 128-byte rows (GK = 64) use row & 7.
template <int GK>
__device__ __forceinline__ int gswz(int row) {
  return GK == 64 ? (row & 7) : ((row >> 2) & 3);
}

// Global -> LDS copy of 16 bytes per lane (lane l's bytes land at
// lds_base + 16 l; lds_base wave-uniform), counted by vmcnt.
__device__ __forceinline__ void gemm_copy16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(
      src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Waits until at most N of this wave's vector memory operations are in
// flight (s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, the other
// counters left at their maxima).
template <int N>
__device__ __forceinline__ void gemm_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8) | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's LDS reads have completed; no fence,
// so copies still in flight are not waited for.
__device__ __forceinline__ void gemm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Element offset of (row, unit) in a staged operand tile.
template <int GK>
__device__ __forceinline__ int goff(int row, int unit) {
  return row * GK + ((unit ^ gswz<GK>(row)) << 3);
}

// Stores the block's BM x BN result tile (wave (wr, wc) holds rows
// wr * WM .., columns wc * WN .. as 16x16 accumulator tiles; lane (g, m) of
// tile (i, j) holds rows 16i + 4g + rr, column 16j + m) into the column
// segments of p.  NT threads take part; smem_raw (smem_bytes long) is free.
template <int BM, int BN, int WM, int WN, int NT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p,
                                              const f32x4 (&acc)[WM / 16][WN / 16],
                                              int64_t m0, int64_t n0, int wr, int wc, int tid,
                                              char* smem_raw, size_t smem_bytes) {
  constexpr int TI = WM / 16, TJ = WN / 16;
  const int lane = tid & 63, g = lane >> 4, m = lane & 15;
  // epilogue.  Through LDS when the destinations allow 16-byte stores and
  // the tile fits the staging area: each wave writes its accumulators as
  // bf16 into a row-major tile, then every thread stores 8 consecutive
  // columns of a row at once -- an eighth of the store instructions of
  // storing each lane's elements where they lie, which (with every block
  // storing at once) took up to 11 us of a 72 us in_proj block.
  constexpr int LDT = BN + 8;  // row pitch of the tile (a 16-byte pad)
  if ((size_t)BM * LDT * 2 <= smem_bytes) {
    if (p.vec_store) {
      __bf16* tile = reinterpret_cast<__bf16*>(smem_raw);
      gemm_barrier();  // every wave is done with the staging slots
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            tile[(wr * WM + 16 * i + 4 * g + rr) * LDT + wc * WN + 16 * j + m] =
                (__bf16)acc[i][j][rr];
      gemm_barrier();
      constexpr int PPR = BN / 8;  // 16-byte pieces per row
      static_assert((BM * PPR) % NT == 0, "pieces must split evenly over the block");
#pragma unroll 4
      for (int q = 0; q < BM * PPR / NT; ++q) {
        const int P = tid + NT * q, row = P / PPR, pc = P % PPR;
        const int64_t r = m0 + row, col = n0 + 8 * pc;
        if (r >= p.M || col >= p.N) continue;
        int s = 0;
#pragma unroll
        for (int t = 1; t < 4; ++t)
          if (t < p.nseg && col >= p.col0[t]) s = t;
        void* const sp = s == 0 ? p.ptr[0] : s == 1 ? p.ptr[1] : s == 2 ? p.ptr[2] : p.ptr[3];
        const int64_t sc0 =
            s == 0 ? p.col0[0] : s == 1 ? p.col0[1] : s == 2 ? p.col0[2] : p.col0[3];
        const int64_t ld = s == 0 ? p.ld[0] : s == 1 ? p.ld[1] : s == 2 ? p.ld[2] : p.ld[3];
        __bf16* dst = reinterpret_cast<__bf16*>(sp) + r * ld + (col - sc0);
        const __bf16* src = tile + row * LDT + 8 * pc;
        if (col + 8 <= p.N) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
          for (int e = 0; e < p.N - col; ++e) dst[e] = src[e];
        }
      }
      return;
    }
  }
  // (otherwise) lane (g, m) of tile (i, j) holds rows 16i + 4g + rr, column
  // 16j + m of the wave tile
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t cb = n0 + wc * WN + 16 * j;  // first column of the group
    if (cb >= p.N) continue;
    // each lane's own column picks its segment (a segment may start inside
    // the group); the segment's fields by selects (an indexed read of the
    // argument arrays would be a vector load)
    const int64_t col = cb + m;
    int s = 0;
#pragma unroll
    for (int t = 1; t < 4; ++t)
      if (t < p.nseg && col >= p.col0[t]) s = t;
    void* const sp = s == 0 ? p.ptr[0] : s == 1 ? p.ptr[1] : s == 2 ? p.ptr[2] : p.ptr[3];
    const int64_t sc0 = s == 0 ? p.col0[0] : s == 1 ? p.col0[1] : s == 2 ? p.col0[2] : p.col0[3];
    __bf16* dst0 = reinterpret_cast<__bf16*>(sp) + (col - sc0);
    const int64_t ld = s == 0 ? p.ld[0] : s == 1 ? p.ld[1] : s == 2 ? p.ld[2] : p.ld[3];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t r0 = m0 + wr * WM + 16 * i + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (r0 + rr < p.M && col < p.N) dst0[(r0 + rr) * ld] = (__bf16)acc[i][j][rr];
    }
  }}

template <int BM, int BN, int GK, int ST>
__global__ __launch_bounds__(256, BM == 256 ? 1 : 2) void gemm_kernel(GemmArgs p) {
  extern __shared__ __align__(1024) char smem_raw[];
  using SM = GemmSmem<BM, BN, GK, ST>;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int KG = GK / 32;                 // k-groups per tile
  constexpr int RU = GK / 8;                  // 16-byte units per staged row
  constexpr int RPC = 64 / RU;                // rows per 1 KB copy
  constexpr int CA = BM / RPC, CB = BN / RPC;  // copies per tile
  constexpr int NC = (CA + CB) / 4;            // per wave
  static_assert((CA + CB) % 4 == 0, "copies must split evenly over 4 waves");
  static_assert((ST - 1) * NC < 64, "copies in flight exceed vmcnt");

  // tile of this block: the row tiles of one column tile share an XCD
  // (blockIdx % 8), so that XCD's L2 serves the column tile's B rows
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r8 = bid >> 3;
  const int mt = r8 % p.mtiles;
  const int nt = (r8 / p.mtiles) * 8 + xcd;
  if (nt >= p.ntiles) return;
  const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
  // the wave index as a scalar, so every copy's LDS address (and M0) is
  // scalar arithmetic
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, m = lane & 15;
  const int wr = w >> 1, wc = w & 1;

  // this wave's copies: c = w, w + 4, ...; copy c < CA stages A rows
  // RPC c .. RPC c + RPC - 1, otherwise B rows; lane l brings row
  // RPC c + l / RU, staged position l % RU, which holds unit
  // (l % RU) ^ swz(row) (the same for every copy, since RPC c is a multiple
  // of the swizzle period).  Rows past the last one are clamped per lane.
  const int lrow = lane / RU;
  const int lunit = (lane % RU) ^ gswz<GK>(lrow);
  // (branch-free, so that the copies form one straight run the scheduler
  // can spread among MFMAs: with CA a multiple of 4, copy q of every wave
  // stages A rows exactly when q < CA / 4, and every lane clamps its row)
  static_assert(CA % 4 == 0, "A copies must split evenly over 4 waves");
  auto issue = [&](int kt) {
    const int st = kt % ST;
    const int64_t kb = (int64_t)kt * GK * 2;  // byte offset of the k-tile
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      constexpr int kQA = CA / 4;
      const bool isA = q < kQA;  // compile-time after unrolling
      const int cc = isA ? w + 4 * q : w + 4 * (q - kQA);
      const int64_t row = isA ? min(m0 + RPC * cc + lrow, p.M - 1)
                              : min(n0 + RPC * cc + lrow, p.N - 1);
      const char* src = isA ? reinterpret_cast<const char*>(p.A + row * p.lda)
                            : reinterpret_cast<const char*>(p.B + row * p.ldb);
      __bf16* dst = isA ? &sm.A[st][cc * 512] : &sm.B[st][cc * 512];
      gemm_copy16(src + kb + lunit * 16, dst);
    }
  };
  // tile kt has landed once at most n_after later tiles' copies are in flight
  auto wait_tiles = [&](int n_after) {
    if (ST > 3 && n_after >= 3)
      gemm_wait_vm<(ST > 3 ? 3 * NC : 0)>();
    else if (ST > 2 && n_after >= 2)
      gemm_wait_vm<(ST > 2 ? 2 * NC : 0)>();
    else if (n_after >= 1)
      gemm_wait_vm<NC>();
    else
      gemm_wait_vm<0>();
  };

  const int KT = (int)(p.K / GK);
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = zero4();

  if constexpr (KG == 2 && ST == 2) {
    // Two k-groups per tile, two slots.  Each half-iteration runs one
    // k-group's products on fragments already in registers while it reads
    // the next k-group's fragments, so LDS latency hides behind the MFMAs:
    //   A(kt): products of k-group 0 of tile kt | read k-group 1 of tile kt
    //   B(kt): tile kt + 1 has landed; barrier (every wave is done reading
    //          tile kt, so its slot takes tile kt + 2);
    //          products of k-group 1 of tile kt | read k-group 0 of tile kt + 1
    // Each copy has one tile-time to land.
    Frag<__bf16> f0a[TI], f0b[TJ], f1a[TI], f1b[TJ];
    auto read_kg = [&](int st, int kk, Frag<__bf16>(&fa)[TI], Frag<__bf16>(&fb)[TJ]) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
        fa[i] = *reinterpret_cast<const Frag<__bf16>*>(
            &sm.A[st][goff<GK>(wr * WM + 16 * i + m, 4 * kk + g)]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        fb[j] = *reinterpret_cast<const Frag<__bf16>*>(
            &sm.B[st][goff<GK>(wc * WN + 16 * j + m, 4 * kk + g)]);
    };
    auto products = [&](const Frag<__bf16>(&fa)[TI], const Frag<__bf16>(&fb)[TJ]) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) mma(acc[i][j], fa[i], fb[j]);
    };
    // interleave: each LDS read of the next k-group between products
    constexpr int NR = TI + TJ, NP = TI * TJ;
    auto interleave = [&]() {
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, NP / NR, 0);  // MFMAs
      }
    };
    // ... and B's copies too: issued in one burst they held back the
    // products behind them (B took 1.7x as long as A); spread out, they
    // drain while the products run
    auto interleave_copies = [&]() {
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
        if (q < NC) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one copy
        __builtin_amdgcn_sched_group_barrier(0x008, NP / NR, 0);  // MFMAs
      }
    };
    if (KT > 0) issue(0);
    if (KT > 1) issue(1);
    if (KT > 1)
      gemm_wait_vm<NC>();
    else
      gemm_wait_vm<0>();
    gemm_barrier();
    if (KT > 0) read_kg(0, 0, f0a, f0b);
    for (int kt = 0; kt < KT; ++kt) {
      const int st = kt & 1;
      // A(kt)
      __builtin_amdgcn_sched_barrier(0);
      products(f0a, f0b);
      read_kg(st, 1, f1a, f1b);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      // B(kt): k-group 1's fragments are needed now (an explicit wait on
      // both paths keeps the compiler from waiting for the reads below)
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      gemm_wait_vm<0>();
      gemm_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // tile kt + 2 into tile kt's slot, free now that every wave has read
      // it; the last two iterations copy tile KT - 1 again (unconditional,
      // so the copies interleave with the products; nothing reads it).
      // (after the last tile the reads below fetch a stale slot, unused)
      issue(min(kt + 2, KT - 1));
      products(f1a, f1b);
      read_kg(st ^ 1, 0, f0a, f0b);
      interleave_copies();
      __builtin_amdgcn_sched_barrier(0);
    }
    gemm_wait_vm<0>();  // the repeated copies, before the block ends
  } else {
    for (int kt = 0; kt < ST - 1 && kt < KT; ++kt) issue(kt);
    // Iteration kt: tile kt has landed (this wave's copies, then everyone's
    // after the barrier; every wave is also done with tile kt - 1, whose
    // slot tile kt + ST - 1 reuses); issue tile kt + ST - 1; read all of
    // tile kt's fragments, then run its products -- the scheduling barrier
    // keeps every read ahead of the products.
    for (int kt = 0; kt < KT; ++kt) {
      wait_tiles(min(kt + ST - 2, KT - 1) - kt);
      gemm_barrier();
      if (kt + ST - 1 < KT) issue(kt + ST - 1);
      const int st = kt % ST;
      Frag<__bf16> af[KG][TI], bfr[KG][TJ];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
          af[kk][i] = *reinterpret_cast<const Frag<__bf16>*>(
              &sm.A[st][goff<GK>(wr * WM + 16 * i + m, 4 * kk + g)]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          bfr[kk][j] = *reinterpret_cast<const Frag<__bf16>*>(
              &sm.B[st][goff<GK>(wc * WN + 16 * j + m, 4 * kk + g)]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KG; ++kk)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) mma(acc[i][j], af[kk][i], bfr[kk][j]);
    }
  }

  gemm_epilogue<BM, BN, WM, WN, 256>(p, acc, m0, n0, wr, wc, tid, smem_raw, sizeof(SM));
}

// Eight waves (two per SIMD) on a 256- or 128-row tile, 64-wide k-tiles in
// S slots: two for 256-row tiles (three would not fit the LDS), three for
// 128-row ones, whose k-tile is too short a step to cover its copies' latency
// from one tile ahead.  With one wave per SIMD, a wave whose copy waits for
// the memory pipeline also holds back the products queued behind it; a
// second wave on the SIMD keeps the matrix unit busy meanwhile.  Waves form a 4 x 2 grid
// of BM / 4-row tiles (BN / 2 columns), so their accumulators and two sets
// of fragments fit the registers a wave has at two waves per SIMD.  The
// staging, swizzle, copy order and half-step structure are those of
// gemm_kernel's two-slot path; each wave issues NC copies per k-tile (the
// surplus copies of the last wave group repeat the last B copy, which
// writes the same bytes to the same place).
template <int BM, int BN, int S = 2>
constexpr size_t gemm8_smem_bytes() {
  constexpr size_t stage = (size_t)S * (BM + BN) * 64 * 2, tile = BM * (BN + 8) * 2;
  return stage > tile ? stage : tile;
}

template <int BM, int BN, int S>
struct Gemm8Smem {
  __bf16 A[S][BM * 64];
  __bf16 B[S][BN * 64];
};

// S slots: tile kt is staged in slot kt % S, S - 1 tiles ahead of its use.
template <int BM, int BN, int S = 2>
__global__ __launch_bounds__(512, BM == 256 ? 1 : 2) void gemm8_kernel(GemmArgs p) {
  extern __shared__ __align__(1024) char smem_raw[];
  constexpr int GK = 64, NW = 8;
  static_assert(S >= 2, "at least two slots");
  using SM = Gemm8Smem<BM, BN, S>;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  constexpr int WM = BM / 4, WN = BN / 2;  // wave tile
  static_assert(WM % 16 == 0, "wave tile rows must be whole 16-row tiles");
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int RU = GK / 8;                   // 16-byte units per staged row
  constexpr int RPC = 64 / RU;                 // rows per 1 KB copy
  constexpr int CA = BM / RPC, CB = BN / RPC;  // copies per tile
  constexpr int NC = (CA + CB + NW - 1) / NW;  // per wave
  constexpr int kQA = CA / NW;
  static_assert(CA % NW == 0, "A copies must split evenly over the waves");
  static_assert(WN % 16 == 0, "wave tile columns must be whole 16-column tiles");
  static_assert(NC * (S - 1) < 64, "copies in flight exceed vmcnt");

  const int bid = blockIdx.x;
  const int xcd = bid & 7, r8 = bid >> 3;
  const int mt = r8 % p.mtiles;
  const int nt = (r8 / p.mtiles) * 8 + xcd;
  if (nt >= p.ntiles) return;
  const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, m = lane & 15;
  const int wr = w >> 1, wc = w & 1;
  const int lrow = lane / RU;
  const int lunit = (lane % RU) ^ gswz<GK>(lrow);
  auto issue = [&](int kt) {
    const int st = kt % S;
    const int64_t kb = (int64_t)kt * GK * 2;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const bool isA = q < kQA;  // compile-time after unrolling
      const int cc = isA ? w + NW * q : min(w + NW * (q - kQA), CB - 1);
      const int64_t row = isA ? min(m0 + RPC * cc + lrow, p.M - 1)
                              : min(n0 + RPC * cc + lrow, p.N - 1);
      const char* src = isA ? reinterpret_cast<const char*>(p.A + row * p.lda)
                            : reinterpret_cast<const char*>(p.B + row * p.ldb);
      __bf16* dst = isA ? &sm.A[st][cc * 512] : &sm.B[st][cc * 512];
      gemm_copy16(src + kb + lunit * 16, dst);
    }
  };

  const int KT = (int)(p.K / GK);
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = zero4();

  Frag<__bf16> f0a[TI], f0b[TJ], f1a[TI], f1b[TJ];
  auto read_kg = [&](int st, int kk, Frag<__bf16>(&fa)[TI], Frag<__bf16>(&fb)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
      fa[i] = *reinterpret_cast<const Frag<__bf16>*>(
          &sm.A[st][goff<GK>(wr * WM + 16 * i + m, 4 * kk + g)]);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      fb[j] = *reinterpret_cast<const Frag<__bf16>*>(
          &sm.B[st][goff<GK>(wc * WN + 16 * j + m, 4 * kk + g)]);
  };
  auto products = [&](const Frag<__bf16>(&fa)[TI], const Frag<__bf16>(&fb)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) mma(acc[i][j], fa[i], fb[j]);
  };
  constexpr int NR = TI + TJ, NP = TI * TJ;
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // one DS read
      __builtin_amdgcn_sched_group_barrier(0x008, NP / NR, 0);  // MFMAs
    }
  };
  auto interleave_copies = [&]() {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                // one DS read
      if (q < NC) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one copy
      __builtin_amdgcn_sched_group_barrier(0x008, NP / NR, 0);         // MFMAs
    }
  };
  // the schedule of gemm_kernel's two-slot path (see there), S - 1 tiles
  // ahead: the prologue stages tiles 0 .. S - 1 (past the last tile the
  // last is staged again, rewriting the same bytes in its own slot, so
  // every step issues the same copies and the vmcnt counts stay fixed)
  if (KT > 0) {
#pragma unroll
    for (int i = 0; i < S; ++i) issue(min(i, KT - 1));
    gemm_wait_vm<NC * (S - 1)>();  // tile 0 has landed
  }
  gemm_barrier();
  if (KT > 0) read_kg(0, 0, f0a, f0b);
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % S;
    __builtin_amdgcn_sched_barrier(0);
    products(f0a, f0b);
    read_kg(st, 1, f1a, f1b);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    gemm_wait_vm<NC * (S - 2)>();       // tiles up to kt + 1 have landed
    gemm_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(min(kt + S, KT - 1));  // into slot kt % S, read by every wave above
    products(f1a, f1b);
    read_kg((kt + 1) % S, 0, f0a, f0b);
    interleave_copies();
    __builtin_amdgcn_sched_barrier(0);
  }
  gemm_wait_vm<0>();
  gemm_epilogue<BM, BN, WM, WN, 512>(p, acc, m0, n0, wr, wc, tid, smem_raw,
                                     gemm8_smem_bytes<BM, BN, S>());
}

// ------------------------------------------------------------ conv1d ----
//
// Depthwise causal conv of width W over C channels, then SiLU:
//   y[t][c] = silu(sum_{j < W} w[c][j] * x[t - (W - 1) + j][c]),
// where a row before the start s of t's sequence n is that sequence's
// history: x[s - d] = hin[n][W - 1 - d] for d = 1 .. W - 1 (zero when no
// history is given).  Tap W - 1 meets the current token.  x rows have
// stride ldx; the channels go to up to three destinations (q | k | v), each
// a dense [T][width] array.
//
// A thread owns 8 channels over a tile of kConvTT tokens: it loads the
// tile's kConvTT + W - 1 rows once (16 bytes each, rows clamped into
// [0, T) so every load is in bounds and unconditional) and its 8 x W
// weights as W 16-byte vectors, then forms each token's W taps from
// registers.  A block is 256 threads = 2048 consecutive channels of one
// token tile, so each row read and each result row written by a wave is
// 1 KB contiguous.  A tile whose taps all lie inside one sequence (every
// tile but those at a sequence start) takes a branch-free path; otherwise
// taps before the token's sequence start take the history row instead
// (block-uniform branches, the start tracked with a block-uniform walk over
// cu).  fp32 arithmetic with the hardware exponential and reciprocal in
// the SiLU, bf16 result.
constexpr int kConvTT = 8;

template <int W>
__global__ __launch_bounds__(256) void conv_silu_kernel(ConvArgs p) {
  const int groups = p.C / 8;
  const int cblocks = (groups + 255) / 256;
  const int cb = blockIdx.x % cblocks;
  const int64_t t0 = (int64_t)(blockIdx.x / cblocks) * kConvTT;
  const int grp = cb * 256 + (int)threadIdx.x;
  const bool live = grp < groups;
  const int c0 = (live ? grp : groups - 1) * 8;
  // rows t0 - (W - 1) .. t0 + kConvTT - 1
  constexpr int R = kConvTT + W - 1;
  uint4 xr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    int64_t row = t0 - (W - 1) + i;
    row = row < 0 ? 0 : (row >= p.T ? p.T - 1 : row);
    xr[i] = *reinterpret_cast<const uint4*>(p.x + row * p.ldx + c0);
  }
  // weights of channels c0..c0+7: 8 * W contiguous bf16, 16-byte aligned
  float wv[8][W];
  {
    const uint4* wp = reinterpret_cast<const uint4*>(p.w + (int64_t)c0 * W);
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const bf16x8 h = __builtin_bit_cast(bf16x8, wp[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int flat = 8 * u + e;
        wv[flat / W][flat % W] = (float)h[e];
      }
    }
  }
  // sequence of token t0: the largest n with cu[n] <= t0
  int lo = 0;
  if (p.cu) {
    int hi = p.N;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu[mid] <= t0)
        lo = mid;
      else
        hi = mid - 1;
    }
  }
  // destination of channel c0, chosen by selects (an indexed read of the
  // argument arrays would become a vector load behind the row loads)
  const bool d1 = c0 >= p.dcol0[1], d2 = c0 >= p.dcol0[2];
  __bf16* const dst = (d2 ? p.dst[2] : d1 ? p.dst[1] : p.dst[0]) +
                      (c0 - (d2 ? p.dcol0[2] : d1 ? p.dcol0[1] : p.dcol0[0]));
  const int64_t dld = d2 ? p.dld[2] : d1 ? p.dld[1] : p.dld[0];
  // every tap of every token of the tile inside the sequence of t0
  bool clean = t0 >= W - 1;
  if (p.cu && clean) {
    const int64_t s = p.cu[lo];
    const int64_t next = lo < p.N ? (int64_t)p.cu[lo + 1] : p.T;
    clean = s <= t0 - (W - 1) && next >= t0 + kConvTT;
  }
  if (clean) {
#pragma unroll
    for (int i = 0; i < kConvTT; ++i) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, xr[i + j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wv[e][j] * (float)xv[e];
      }
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = silu_fast(acc[e]);
      const int64_t t = t0 + i;
      if (live && t < p.T) store_packed(dst + t * dld, y);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kConvTT; ++i) {
    const int64_t t = t0 + i;
    int64_t s = 0;
    if (p.cu) {
      while (lo < p.N && p.cu[lo + 1] <= t) ++lo;
      s = p.cu[lo] < 0 ? 0 : p.cu[lo];
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const int64_t tt = t - (W - 1) + j;
      uint4 raw = xr[i + j];
      if (tt < s) {  // history row W - 1 - (s - tt) of sequence lo
        raw = uint4{0u, 0u, 0u, 0u};
        // (the clamps only matter for tokens past T and malformed cu)
        const int64_t hr = (W - 1) - (s - tt);
        const int64_t hn = lo < p.N ? lo : p.N - 1;
        if (p.hin && hr >= 0)
          raw = *reinterpret_cast<const uint4*>(p.hin + (hn * (W - 1) + hr) * p.C + c0);
      }
      const bf16x8 xv = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wv[e][j] * (float)xv[e];
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = silu_fast(acc[e]);
    if (live && t < p.T) store_packed(dst + t * dld, y);
  }
}

// New history of each sequence: its last W - 1 input rows, taken from the
// history given on entry where the sequence is shorter than that.  One
// thread per (sequence, 8 channels) reads every row it needs before it
// writes, so hout may be hin.
__global__ __launch_bounds__(256) void conv_history_kernel(ConvArgs p) {
  const int groups = p.C / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.N * groups) return;
  const int n = (int)(idx / groups);
  const int c0 = (int)(idx % groups) * 8;
  const int H = p.W - 1;
  int64_t s = 0, e = p.T;
  if (p.cu) {
    s = p.cu[n];
    e = p.cu[n + 1];
    s = s < 0 ? 0 : (s > p.T ? p.T : s);
    e = e < s ? s : (e > p.T ? p.T : e);
  }
  const int64_t len = e - s;
  uint4 rows[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    rows[j] = uint4{0u, 0u, 0u, 0u};
    if (j < H) {
      const int64_t pos = len - H + j;  // index within the sequence
      if (pos >= 0)
        rows[j] = *reinterpret_cast<const uint4*>(p.x + (s + pos) * p.ldx + c0);
      else if (p.hin)
        rows[j] = *reinterpret_cast<const uint4*>(p.hin + ((int64_t)n * H + H + pos) * p.C + c0);
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < H) *reinterpret_cast<uint4*>(p.hout + ((int64_t)n * H + j) * p.C + c0) = rows[j];
}

// ------------------------------------------------------------ MFMA probe ----
//
// Measurement only: the bf16 MFMA rate this device sustains.  Every wave
// runs `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16 on
// register operands (no memory traffic in the loop) and writes one float
// per lane so the work cannot be dropped.  FLOP = 2 * 16 * 16 * 32 * 8 *
// iters per wave.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int64_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  Frag<__bf16> a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a.v[j] = (__bf16)(0.001f * (float)(lane + j));
    b.v[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = zero4();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) mma(acc[u], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_mfma_probe(int64_t iters, int blocks, float* out, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, out);
  return hipGetLastError();
}

// ------------------------------------------------------------- launches ----

static hipError_t allow_lds_once(const void* fn, size_t bytes, unsigned long long* mask) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const unsigned long long bit = 1ull << (dev & 63);
  if (__atomic_load_n(mask, __ATOMIC_ACQUIRE) & bit) return hipSuccess;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess) __atomic_fetch_or(mask, bit, __ATOMIC_RELEASE);
  return err;
}

template <int BM, int BN, int GK, int ST>
static hipError_t launch_gemm_tiles(GemmArgs a, hipStream_t st) {
  static unsigned long long mask = 0ull;
  const size_t smem = sizeof(GemmSmem<BM, BN, GK, ST>);
  hipError_t err = allow_lds_once((const void*)gemm_kernel<BM, BN, GK, ST>, smem, &mask);
  if (err != hipSuccess) return err;
  a.mtiles = (int)((a.M + BM - 1) / BM);
  a.ntiles = (int)((a.N + BN - 1) / BN);
  const int64_t blocks = (int64_t)((a.ntiles + 7) / 8) * 8 * a.mtiles;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, GK, ST>), dim3((unsigned)blocks), dim3(256), smem, st,
                     a);
  return hipGetLastError();
}

template <int BM, int BN, int S = 2>
static hipError_t launch_gemm8(GemmArgs a, hipStream_t st) {
  static unsigned long long mask = 0ull;
  constexpr size_t smem = gemm8_smem_bytes<BM, BN, S>();
  hipError_t err = allow_lds_once((const void*)gemm8_kernel<BM, BN, S>, smem, &mask);
  if (err != hipSuccess) return err;
  a.mtiles = (int)((a.M + BM - 1) / BM);
  a.ntiles = (int)((a.N + BN - 1) / BN);
  const int64_t blocks = (int64_t)((a.ntiles + 7) / 8) * 8 * a.mtiles;
  hipLaunchKernelGGL((gemm8_kernel<BM, BN, S>), dim3((unsigned)blocks), dim3(512), smem, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a0, hipStream_t st) {
  if (a0.M <= 0 || a0.N <= 0) return hipSuccess;
  GemmArgs a = a0;
  a.vec_store = 1;
  for (int s = 0; s < a.nseg && s < 4; ++s)
    if ((reinterpret_cast<uintptr_t>(a.ptr[s]) & 15) != 0 || a.ld[s] % 8 != 0 ||
        a.col0[s] % 8 != 0)
      a.vec_store = 0;
  // large tiles when they still give every CU a block; otherwise smaller
  // ones for more blocks.  k-tiles of 64 (whole 128-byte rows; two slots for
  // 256-row tiles, three for 128-row ones) when K allows, else 32 (four
  // slots).
  const int64_t big = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  const bool k64 = a.K % 64 == 0;
  if (big >= 256) {
    if (!k64) return launch_gemm_tiles<256, 256, 32, 4>(a, st);
    // one block per CU: pick the column width whose rounds of 256 blocks
    // waste the least tile area (e.g. 2048 x 12352: 256-wide tiles make
    // 392 blocks, 1.53 rounds; 224-wide ones 448 blocks, 1.75 rounds)
    const int64_t mt = (a.M + 255) / 256;
    auto cost = [&](int64_t bn) {
      const int64_t tiles = mt * ((a.N + bn - 1) / bn);
      return ((tiles + 255) / 256) * bn;
    };
    const int64_t c256 = cost(256), c224 = cost(224), c192 = cost(192);
    if (c224 < c256 && c224 <= c192) return launch_gemm8<256, 224>(a, st);
    if (c192 < c256) return launch_gemm8<256, 192>(a, st);
    return launch_gemm8<256, 256>(a, st);
  }
  if (!k64) return launch_gemm_tiles<128, 128, 32, 4>(a, st);
  // 128-row tiles, the same cost per round of 256 blocks (e.g. 2048 x
  // 2560: 128-wide tiles make 320 blocks, two rounds on the CUs that take a
  // second one; 160-wide ones exactly 256)
  const int64_t mt = (a.M + 127) / 128;
  auto cost = [&](int64_t bn) {
    const int64_t tiles = mt * ((a.N + bn - 1) / bn);
    return ((tiles + 255) / 256) * bn;
  };
  if (cost(160) < cost(128)) return launch_gemm8<128, 160, 3>(a, st);
  return launch_gemm8<128, 128, 3>(a, st);
}

hipError_t launch_conv_silu(const ConvArgs& a, hipStream_t st) {
  if (a.C == 0) return hipSuccess;
  if (a.W < 1 || a.W > 4) return hipErrorInvalidValue;
  if (a.T > 0) {
    const int64_t cblocks = (a.C / 8 + 255) / 256;
    const unsigned blocks = (unsigned)(cblocks * ((a.T + kConvTT - 1) / kConvTT));
    switch (a.W) {
      case 1: hipLaunchKernelGGL(conv_silu_kernel<1>, dim3(blocks), dim3(256), 0, st, a); break;
      case 2: hipLaunchKernelGGL(conv_silu_kernel<2>, dim3(blocks), dim3(256), 0, st, a); break;
      case 3: hipLaunchKernelGGL(conv_silu_kernel<3>, dim3(blocks), dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL(conv_silu_kernel<4>, dim3(blocks), dim3(256), 0, st, a); break;
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return launch_conv_history(a, st);
}

hipError_t launch_conv_history(const ConvArgs& a, hipStream_t st) {
  if (a.hout && a.W > 1 && a.N > 0 && a.C > 0) {
    const int64_t n = (int64_t)a.N * (a.C / 8);
    hipLaunchKernelGGL(conv_history_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdn
