// gdn_decode.hpp -- host-side launch description of the decode step and
// the short-prefill launcher, shared by the C ABI layer and the recurrent
// kernels' launchers.  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.hpp"

namespace gdn {

// One recurrent step per request on a slot-addressed state cache.
struct DecodeLaunch {
  int dtype;  // 0 = fp32, 1 = bf16
  int B, Hk, Hv;
  float scale, l2_eps, norm_eps;
  const void *q, *k, *v, *a, *b, *z;
  const float *A_log, *dt_bias, *norm_w;
  float* cache;          // [num_slots][Hv][128][128]
  const int32_t* slots;  // [B] or null (request i uses slot i)
  int64_t num_slots;
  void* o;
};

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);

// A whole prefill call (see PrefillLaunch) as the recurrence token by token
// in one kernel, one block per (sequence, value head), for calls with few
// tokens; uses no workspace.
// stage_events as launch_prefill (the kernel is stage kStageShort)
hipError_t launch_short_prefill(const PrefillLaunch& p, hipStream_t stream,
                                hipEvent_t* stage_events, unsigned* stage_ran);

}  // namespace gdn
