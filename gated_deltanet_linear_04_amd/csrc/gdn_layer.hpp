// gdn_layer.hpp -- host-side launch descriptions of the full layer's
// kernels (projection GEMM, conv1d + SiLU), shared by the C ABI layer and
// their launchers.  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// C[M][N] = A[M][K] * B[N][K]^T (bf16, fp32 accumulation, bf16 result),
// columns split over up to four destinations (segment s: columns
// [col0[s], col0[s + 1]) -> ptr[s] + row * ld[s] + (col - col0[s])).
struct GemmArgs {
  const __bf16* A;
  const __bf16* B;
  int64_t lda, ldb, M, N, K;
  int nseg;
  int64_t col0[4];
  void* ptr[4];
  int64_t ld[4];
  int mtiles, ntiles;  // set by the launcher
  // set by the launcher: every destination allows 16-byte stores of 8
  // consecutive columns (16-byte aligned base, row stride a multiple of 8)
  int vec_store;
};

// Depthwise causal conv (width W) + SiLU of x [T][C] (row stride ldx);
// channels go to up to three dense destinations (dst[d] covers channels
// [dcol0[d], dcol0[d + 1])).  Before each sequence's first token the conv
// sees that sequence's history rows hin[n][0 .. W - 2][C] (oldest first), or
// zeros when hin is null.
struct ConvArgs {
  const __bf16* x;
  int64_t ldx;
  const __bf16* w;  // [C][W]
  int W;
  int64_t T;
  int C;
  const int32_t* cu;  // [N + 1] or null (one sequence)
  int N;
  __bf16* dst[3];
  int64_t dld[3];
  int dcol0[3];
  const __bf16* hin;  // [N][W - 1][C] or null
  __bf16* hout;       // [N][W - 1][C] or null: the last W - 1 input rows
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// The conv, then (when hout is given) the new history rows in a second
// launch, so that hout may alias hin.
hipError_t launch_conv_silu(const ConvArgs& a, hipStream_t stream);
// The new history rows alone (hout given; W > 1).
hipError_t launch_conv_history(const ConvArgs& a, hipStream_t stream);

// Measurement only: `blocks` blocks of 256 threads each run iters rounds of
// eight bf16 MFMAs per wave; out holds blocks * 256 floats.
hipError_t launch_mfma_probe(int64_t iters, int blocks, float* out, hipStream_t stream);

}  // namespace gdn
