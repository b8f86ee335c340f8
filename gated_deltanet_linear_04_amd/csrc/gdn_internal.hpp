// gdn_internal.hpp -- host-side plan shared by the C ABI layer and the
// kernel launchers.  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kHeadDim = 128;  // dk = dv on the GPU path
constexpr int kDvBlock = 16;   // state columns per chain wave
constexpr int kDvBlocks = kHeadDim / kDvBlock;

// Packed-fragment sizes (elements) of the per-chunk intermediates.
constexpr int kFragElems = 64 * 8;                  // one k-group fragment
constexpr int kTbFrags = (kChunk / 16) * (kChunk / 32);  // 64x64 -> 8
constexpr int kScalars = 4;  // ek, fk, fq, eL per token

// Byte offsets of the workspace regions for one call.
struct WorkspaceLayout {
  size_t tb;           // elem [max_chunks][hv][kTbFrags][64][8]
  size_t mp;           // elem [max_chunks][hv][kTbFrags][64][8]
  size_t scal;         // f32  [max_chunks][hv][kScalars][64]
  size_t hc;           // elem [max_chunks][hv][kDvBlocks][4][64][8]
  size_t vp;           // elem [max_chunks][hv][kDvBlocks][2][64][8]
  size_t total;
  int64_t max_chunks;  // workspace chunk slots: ceil(T / 64) + N
};

// Everything one launch sequence needs, with device pointers resolved.
struct PrefillLaunch {
  int dtype;  // 0 = fp32, 1 = bf16
  int N;
  int64_t T;
  int Hk, Hv;
  float scale, l2_eps, norm_eps;
  const void *q, *k, *v, *a, *b, *z;
  const float *A_log, *dt_bias, *norm_w, *state_in;
  const int32_t* cu_seqlens;
  void* o;
  float* state_out;
  char* ws;
  WorkspaceLayout lay;
};

// Optional per-stage event recording (measurement only).
struct StageEvents {
  hipEvent_t* ev;  // [n_stages + 1] or nullptr
};

constexpr int kNumStages = 3;  // prep, chain, out

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream,
                          hipEvent_t* stage_events);

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
};

// Depthwise causal conv (width W, no history before each sequence) + SiLU
// of x [T][C] (row stride ldx); channels go to up to three dense
// destinations (dst[d] covers channels [dcol0[d], dcol0[d + 1])).
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
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_conv_silu(const ConvArgs& a, hipStream_t stream);

}  // namespace gdn
