// gdn_internal.hpp -- host-side plan shared by the C ABI layer and the
// kernel launchers.  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

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
  size_t seg_S, seg_B, seg_M;  // f32 [scan segments][hv][128][128] each (one sequence)
  size_t total;
  int64_t max_chunks;  // workspace chunk slots: ceil(T / 64) + N
};

// The layer's causal conv + SiLU, applied by the prep kernel to the rows it
// stages (bf16 only): x holds the pre-conv q | k | v channels (row stride
// ldx, C = 2 hk dk + hv dv channels, taps w[C][W]); hin the W - 1 rows before
// each sequence's first token ([N][W - 1][C], or null for zeros).  prep
// writes the post-conv rows the other kernels read to the q, k, v pointers of
// the launch (dense [T][hk dk], [T][hk dk], [T][hv dv]).
struct PrepConv {
  const void* x;
  int64_t ldx;
  const void* w;
  const void* hin;
  int W, C;
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
  // sequence-parallel scan of the state chain (one sequence): scan_segments
  // segments of seg_chunks chunks, or scan_segments < 2 for one pass
  int scan_segments, seg_chunks;
  // the layer's conv fused into prep (q, k, v above are then its outputs),
  // or null
  const PrepConv* conv;
};

constexpr int kNumStages = 4;  // prep, chain, out (chunked); short
constexpr int kStageShort = 3;

// stage_events (measurement only): nullptr, or 2 * kNumStages events, the
// start and end of each stage's kernel, attached to its dispatch.
// stage_ran (with stage_events): bit s is cleared for each stage s the call
// does not run, whose events are then left unrecorded.

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream,
                          hipEvent_t* stage_events, unsigned* stage_ran);

// Work-items of the largest grid launch_prefill makes for these sizes (the
// dispatch packet holds a grid's size in work-items as a 32-bit count, so
// the caller rejects calls past 2^32 - 1 before launching anything).
uint64_t prefill_grid_work_items(int64_t max_chunks, int64_t N, int Hk, int Hv,
                                 int scan_segments);

// Workspace of gdn_prefill_noalloc: a static device array of this many bytes
// per GPU.  noalloc_scratch returns its device address on the current
// device (looked up on the first call for that device, then kept).
constexpr size_t kNoAllocScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

}  // namespace gdn
