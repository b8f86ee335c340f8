// gdn_api.cpp -- the C ABI of libgdn.so: argument validation, workspace
// planning and per-stage timing around the kernel launches.
//
// Validation happens entirely on the host before anything is launched, so
// every error path can be exercised without a GPU (the library loads on a
// machine without one; only launches need a device).  Unsupported shapes
// are reported, never silently rerouted -- "feat(qwen35): add SM120
// FlashInfer GDN prefill candidate" (pegainfer PR #862), reviews: unsupported
// shapes and configurations handled explicitly behind a stable C ABI.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/gdn.h"
#include "gdn_decode.hpp"
#include "gdn_internal.hpp"
#include "gdn_layer.hpp"

namespace {

thread_local char g_err[512] = "";

gdn_status fail(gdn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Overflow-checked a * b (returns false on overflow).
bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

// Shape checks shared by the size query and the call.
gdn_status check_desc(const gdn_desc* d) {
  if (!d) return fail(GDN_ERR_INVALID, "desc is NULL");
  if (d->num_seqs < 1) return fail(GDN_ERR_INVALID, "num_seqs must be >= 1");
  if (d->total_tokens < 0)
    return fail(GDN_ERR_INVALID, "total_tokens must be >= 0");
  if (d->total_tokens > INT32_MAX - 64)
    return fail(GDN_ERR_UNSUPPORTED, "total_tokens above 2^31 - 65");
  if (d->hq < 1 || d->hk < 1 || d->hv < 1)
    return fail(GDN_ERR_INVALID, "head counts must be >= 1");
  if (d->hv % d->hk != 0)
    return fail(GDN_ERR_INVALID, "hv (%d) must be a multiple of hk (%d)",
                d->hv, d->hk);
  if (d->dk < 1 || d->dv < 1)
    return fail(GDN_ERR_INVALID, "head dims must be >= 1");
  if (d->dtype != GDN_F32 && d->dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID, "unknown dtype %d", d->dtype);
  if (!isfinite(d->scale) || !isfinite(d->qk_l2_eps) ||
      !isfinite(d->norm_eps) || d->qk_l2_eps < 0.f || d->norm_eps < 0.f)
    return fail(GDN_ERR_INVALID, "scale/eps must be finite, eps >= 0");
  if (d->hq != d->hk)
    return fail(GDN_ERR_UNSUPPORTED, "hq (%d) != hk (%d) is not implemented",
                d->hq, d->hk);
  if (d->dk != gdn::kHeadDim || d->dv != gdn::kHeadDim)
    return fail(GDN_ERR_UNSUPPORTED,
                "head dims dk=%d dv=%d: the GPU path implements 128 x 128",
                d->dk, d->dv);
  if ((int64_t)d->num_seqs * d->hv > (int64_t)INT32_MAX / 16)
    return fail(GDN_ERR_UNSUPPORTED, "num_seqs * hv too large");
  if (d->short_tokens < 0)
    return fail(GDN_ERR_INVALID, "short_tokens must be >= 0");
  if (d->chain_segments < 0)
    return fail(GDN_ERR_INVALID, "chain_segments must be >= 0");
  if (d->chain_segments > 1 && d->num_seqs != 1)
    return fail(GDN_ERR_UNSUPPORTED,
                "chain_segments > 1 scans a single sequence (num_seqs = %d)", d->num_seqs);
  return GDN_OK;
}

// Segments of the sequence-parallel scan of the state chain for `d` (a
// checked descriptor): 1 for one pass, else G >= 2 with seg_chunks chunks
// each (the last may be shorter).  The usual choice (chain_segments 0)
// scans a single sequence when pass A's blocks (Hv x 8 column blocks x (2G
// - 3)) fit the chain's blocks in flight (two per CU for bf16, one for fp32)
// with G >= 3 and at least 8 chunks per segment.
int scan_segments(const gdn_desc* d, int* seg_chunks) {
  *seg_chunks = 0;
  if (d->num_seqs != 1 || d->chain_segments == 1) return 1;
  const int64_t nch = (d->total_tokens + gdn::kChunk - 1) / gdn::kChunk;
  int64_t G = d->chain_segments;
  if (G == 0) {
    const int64_t in_flight = d->dtype == GDN_BF16 ? 512 : 256;
    const int64_t per_seg = (int64_t)d->hv * gdn::kDvBlocks;
    G = (in_flight / per_seg + 3) / 2;
    if (G > nch / 8) G = nch / 8;
    if (G < 3) return 1;
  }
  if (G > 64) G = 64;
  if (G > nch) G = nch;
  if (G < 2) return 1;
  const int64_t sc = (nch + G - 1) / G;
  G = (nch + sc - 1) / sc;
  if (G < 2) return 1;
  *seg_chunks = (int)sc;
  return (int)G;
}

// A launch's grid is at most 2^32 - 1 work-items (the dispatch packet's
// 32-bit grid size); larger calls are refused before anything launches.
gdn_status check_grid(uint64_t work_items, const char* what) {
  if (work_items > 0xFFFFFFFFull)
    return fail(GDN_ERR_UNSUPPORTED,
                "%s: a grid of %llu work-items exceeds 2^32 - 1 (split the call)", what,
                (unsigned long long)work_items);
  return GDN_OK;
}

// Workspace regions, each 256-byte aligned.  Returns false on overflow.
bool plan_workspace(const gdn_desc* d, gdn::WorkspaceLayout* lay) {
  const size_t esz = d->dtype == GDN_BF16 ? 2 : 4;
  const int64_t max_chunks =
      (d->total_tokens + gdn::kChunk - 1) / gdn::kChunk + d->num_seqs;
  if (max_chunks > INT32_MAX) return false;
  lay->max_chunks = max_chunks;
  size_t off = 0, sz = 0;
  size_t per_vhead, per_scal, mc = (size_t)max_chunks;
  if (!mul_ok(mc * (size_t)gdn::kTbFrags * gdn::kFragElems, esz, &per_vhead))
    return false;
  if (!mul_ok(per_vhead, (size_t)d->hv, &sz)) return false;
  lay->tb = off;
  off = align_up(off + sz, 256);
  lay->mp = off;
  off = align_up(off + sz, 256);
  if (!mul_ok(mc * (size_t)gdn::kScalars * gdn::kChunk, 4, &per_scal))
    return false;
  if (!mul_ok(per_scal, (size_t)d->hv, &sz)) return false;
  lay->scal = off;
  off = align_up(off + sz, 256);
  // exported chain state (4 k-group fragments per 16-column block) and delta
  // writes (2 fragments per block): per (slot, value head) 128x128 and
  // 64x128 elements
  size_t per_hc;
  if (!mul_ok(mc * (size_t)gdn::kDvBlocks * 4 * gdn::kFragElems, esz, &per_hc))
    return false;
  if (!mul_ok(per_hc, (size_t)d->hv, &sz)) return false;
  lay->hc = off;
  off = align_up(off + sz, 256);
  lay->vp = off;
  off = align_up(off + sz / 2, 256);
  // start states and maps of the scan's segments
  int seg_chunks = 0;
  const int G = scan_segments(d, &seg_chunks);
  size_t seg_bytes = 0;
  if (G >= 2 &&
      !mul_ok((size_t)G * d->hv, (size_t)gdn::kHeadDim * gdn::kHeadDim * 4, &seg_bytes))
    return false;
  lay->seg_S = off;
  off = align_up(off + seg_bytes, 256);
  lay->seg_B = off;
  off = align_up(off + seg_bytes, 256);
  lay->seg_M = off;
  off = align_up(off + seg_bytes, 256);
  lay->total = off;
  return true;
}

// ---- short prefills ----
// A call of at most L + 2 (N - 1) tokens in all (N sequences, L =
// d->short_tokens; 0 turns this off) runs the recurrence token by token in
// one kernel instead of the three chunked kernels, whose fixed cost
// dominates at a few tokens.  Measured on the 4B geometry: the recurrent
// kernel takes about 3.7 us + 1.7 us per token of its longest sequence, the
// chunked kernels about 17 us + 3.6 us per sequence past the first, so even
// with every token in one sequence the recurrent form is the faster one
// below the usual bound of 8.
constexpr int32_t kShortTokensDefault = 8;

bool short_applies(const gdn_desc* d) {
  const int64_t L = d->short_tokens;
  return L > 0 && (int64_t)d->num_seqs * d->hv <= ((int64_t)1 << 30) &&
         d->total_tokens <= L + 2 * ((int64_t)d->num_seqs - 1);
}

// ---- per-stage timing (measurement only) ----
struct StageTimer {
  std::vector<hipEvent_t> ev;  // max_calls * kNumStages * 2 (start, end)
  std::vector<unsigned> ran;   // per call: bit s set when stage s ran
  int max_calls = 0;
  int calls = 0;
};
thread_local StageTimer g_timer;

void timer_release() {
  for (hipEvent_t e : g_timer.ev) (void)hipEventDestroy(e);
  g_timer.ev.clear();
  g_timer.ran.clear();
  g_timer.max_calls = 0;
  g_timer.calls = 0;
}

// Byte offsets of the full layer's workspace regions.
struct LayerLayout {
  size_t P, z, b, a, q, k, v, y, op, total;
  int64_t Wq, Wv, Wp;  // widths: hk*dk, hv*dv, packed projection
};

gdn_status check_layer(const gdn_layer_desc* d) {
  if (!d) return fail(GDN_ERR_INVALID, "layer desc is NULL");
  gdn_status st = check_desc(&d->op);
  if (st != GDN_OK) return st;
  if (d->op.dtype != GDN_BF16)
    return fail(GDN_ERR_UNSUPPORTED, "the layer path implements bf16 only");
  if (d->hidden < 1) return fail(GDN_ERR_INVALID, "hidden must be >= 1");
  if (d->hidden % 32 != 0)
    return fail(GDN_ERR_UNSUPPORTED, "hidden (%d) must be a multiple of 32",
                d->hidden);
  if (d->conv_width < 1 || d->conv_width > 4)
    return fail(GDN_ERR_UNSUPPORTED, "conv_width (%d) must be in 1..4",
                d->conv_width);
  if (d->conv_fused != 0 && d->conv_fused != 1)
    return fail(GDN_ERR_INVALID, "conv_fused must be 0 or 1");
  return GDN_OK;
}

bool plan_layer(const gdn_layer_desc* d, LayerLayout* L) {
  const size_t T = (size_t)d->op.total_tokens;
  L->Wq = (int64_t)d->op.hk * d->op.dk;
  L->Wv = (int64_t)d->op.hv * d->op.dv;
  L->Wp = 2 * L->Wq + 2 * L->Wv + 2 * d->op.hv;
  size_t off = 0, sz;
  auto region = [&](size_t cols, size_t* at) {
    if (!mul_ok(T, cols * 2, &sz)) return false;
    *at = off;
    off = align_up(off + sz, 256);
    return true;
  };
  if (!region((size_t)(2 * L->Wq + L->Wv), &L->P) || !region((size_t)L->Wv, &L->z) ||
      !region((size_t)d->op.hv, &L->b) || !region((size_t)d->op.hv, &L->a) ||
      !region((size_t)L->Wq, &L->q) || !region((size_t)L->Wq, &L->k) ||
      !region((size_t)L->Wv, &L->v) || !region((size_t)L->Wv, &L->y))
    return false;
  gdn::WorkspaceLayout lay;
  if (!plan_workspace(&d->op, &lay)) return false;
  L->op = off;
  L->total = off + lay.total;
  return true;
}

const char* const kStageNames[gdn::kNumStages] = {"prep", "chain", "out", "short"};

// The prefill behind gdn_prefill and gdn_prefill_noalloc: validation, then
// the launches on the given workspace.
gdn_status prefill_impl(const gdn_desc* d, const void* q, const void* k, const void* v,
                        const void* a, const void* b, const float* A_log,
                        const float* dt_bias, const void* z, const float* norm_w,
                        const float* state_in, const int32_t* cu_seqlens, void* o,
                        float* state_out, void* workspace, size_t workspace_bytes,
                        void* stream, const gdn::PrepConv* conv = nullptr);

}  // namespace

extern "C" {

gdn_status gdn_desc_init(gdn_desc* d, int32_t num_seqs, int64_t total_tokens,
                         int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                         int32_t dtype) {
  if (!d) return fail(GDN_ERR_INVALID, "desc is NULL");
  memset(d, 0, sizeof(*d));
  d->num_seqs = num_seqs;
  d->total_tokens = total_tokens;
  d->hq = hk;
  d->hk = hk;
  d->hv = hv;
  d->dk = dk;
  d->dv = dv;
  d->dtype = dtype;
  d->scale = dk > 0 ? 1.0f / sqrtf((float)dk) : 1.0f;
  d->qk_l2_eps = 1e-6f;
  d->norm_eps = 1e-6f;
  d->short_tokens = kShortTokensDefault;
  return GDN_OK;
}

size_t gdn_prefill_workspace_size(const gdn_desc* d) {
  if (check_desc(d) != GDN_OK) return 0;
  gdn::WorkspaceLayout lay;
  if (!plan_workspace(d, &lay)) return 0;
  return lay.total;
}

gdn_status gdn_prefill(const gdn_desc* d, const void* q, const void* k,
                       const void* v, const void* a, const void* b,
                       const float* A_log, const float* dt_bias, const void* z,
                       const float* norm_w, const float* state_in,
                       const int32_t* cu_seqlens, void* o, float* state_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  return prefill_impl(d, q, k, v, a, b, A_log, dt_bias, z, norm_w, state_in, cu_seqlens, o,
                      state_out, workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_noalloc(const gdn_desc* d, const void* q, const void* k,
                               const void* v, const void* a, const void* b,
                               const float* A_log, const float* dt_bias, const void* z,
                               const float* norm_w, const float* state_in,
                               const int32_t* cu_seqlens, void* o, float* state_out,
                               void* stream) {
  g_err[0] = '\0';
  gdn_status st = check_desc(d);
  if (st != GDN_OK) return st;
  gdn::WorkspaceLayout lay;
  if (!plan_workspace(d, &lay))
    return fail(GDN_ERR_UNSUPPORTED, "workspace size overflows");
  if (lay.total > gdn::kNoAllocScratchBytes)
    return fail(GDN_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; gdn_prefill_noalloc holds %zu "
                "(use gdn_prefill with a workspace)", lay.total, gdn::kNoAllocScratchBytes);
  // the scratch is the current device's array, so the kernels must run there
  int cur = 0;
  hipError_t err = hipGetDevice(&cur);
  if (err != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (stream) {
    hipDevice_t sdev = 0;
    err = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (err != hipSuccess)
      return fail(GDN_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(err));
    if (sdev != cur)
      return fail(GDN_ERR_INVALID,
                  "stream belongs to device %d but device %d is current: the scratch "
                  "array used is the current device's", (int)sdev, cur);
  }
  void* scratch = nullptr;
  err = gdn::noalloc_scratch(&scratch);
  if (err != hipSuccess)
    return fail(GDN_ERR_HIP, "scratch address: %s", hipGetErrorString(err));
  return prefill_impl(d, q, k, v, a, b, A_log, dt_bias, z, norm_w, state_in, cu_seqlens, o,
                      state_out, scratch, gdn::kNoAllocScratchBytes, stream);
}

}  // extern "C"

namespace {

gdn_status prefill_impl(const gdn_desc* d, const void* q, const void* k, const void* v,
                        const void* a, const void* b, const float* A_log,
                        const float* dt_bias, const void* z, const float* norm_w,
                        const float* state_in, const int32_t* cu_seqlens, void* o,
                        float* state_out, void* workspace, size_t workspace_bytes,
                        void* stream, const gdn::PrepConv* conv) {
  gdn_status st = check_desc(d);
  if (st != GDN_OK) return st;
  if (!cu_seqlens && d->num_seqs != 1)
    return fail(GDN_ERR_INVALID, "cu_seqlens is NULL but num_seqs = %d",
                d->num_seqs);
  // with no tokens there is no z row to read, so an empty z may be NULL
  if ((z == nullptr) != (norm_w == nullptr) &&
      !(d->total_tokens == 0 && z == nullptr))
    return fail(GDN_ERR_INVALID, "z and norm_w must both be given or both NULL");
  if (!A_log || !dt_bias) return fail(GDN_ERR_INVALID, "A_log/dt_bias is NULL");
  if (d->total_tokens > 0 && (!q || !k || !v || !a || !b || !o))
    return fail(GDN_ERR_INVALID, "a token tensor (q, k, v, a, b, o) is NULL");
  const void* vec_ptrs[] = {q, k, v, z, o, state_in, state_out};
  const char* vec_names[] = {"q", "k", "v", "z", "o", "state_in", "state_out"};
  for (int i = 0; i < 7; ++i)
    if (vec_ptrs[i] && !aligned(vec_ptrs[i], 16))
      return fail(GDN_ERR_INVALID, "%s is not 16-byte aligned", vec_names[i]);
  const size_t esz = d->dtype == GDN_BF16 ? 2 : 4;
  if ((a && !aligned(a, esz)) || (b && !aligned(b, esz)) ||
      !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
      (norm_w && !aligned(norm_w, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
    return fail(GDN_ERR_INVALID, "a, b, A_log, dt_bias, norm_w or cu_seqlens "
                                 "is misaligned for its element type");
  if (state_in && state_out && state_in != state_out) {
    const size_t bytes = (size_t)d->num_seqs * d->hv * d->dv * d->dk * 4;
    const char* i0 = reinterpret_cast<const char*>(state_in);
    const char* o0 = reinterpret_cast<const char*>(state_out);
    if (i0 < o0 + bytes && o0 < i0 + bytes)
      return fail(GDN_ERR_INVALID, "state_in and state_out partially overlap");
  }
  gdn::WorkspaceLayout lay;
  if (!plan_workspace(d, &lay))
    return fail(GDN_ERR_UNSUPPORTED, "workspace size overflows");
  if (!workspace || workspace_bytes < lay.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                lay.total, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256))
    return fail(GDN_ERR_INVALID, "workspace is not 256-byte aligned");

  gdn::PrefillLaunch p;
  p.dtype = d->dtype == GDN_BF16 ? 1 : 0;
  p.N = d->num_seqs;
  p.T = d->total_tokens;
  p.Hk = d->hk;
  p.Hv = d->hv;
  p.scale = d->scale;
  p.l2_eps = d->qk_l2_eps;
  p.norm_eps = d->norm_eps;
  p.q = q;
  p.k = k;
  p.v = v;
  p.a = a;
  p.b = b;
  p.z = z;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.norm_w = norm_w;
  p.state_in = state_in;
  p.cu_seqlens = cu_seqlens;
  p.o = o;
  p.state_out = state_out;
  p.ws = static_cast<char*>(workspace);
  p.lay = lay;
  p.scan_segments = scan_segments(d, &p.seg_chunks);
  p.conv = conv;

  const bool single = short_applies(d);
  // (the layer only fuses its conv into the chunked kernels)
  if (single && conv)
    return fail(GDN_ERR_INVALID, "internal: fused conv on the single-kernel form");
  st = check_grid(single ? (uint64_t)d->num_seqs * (uint64_t)d->hv * 256
                         : gdn::prefill_grid_work_items(lay.max_chunks, d->num_seqs, d->hk,
                                                        d->hv, p.scan_segments),
                  "prefill");
  if (st != GDN_OK) return st;

  hipEvent_t* ev = nullptr;
  unsigned* ran = nullptr;
  if (g_timer.max_calls > 0 && g_timer.calls < g_timer.max_calls) {
    ev = &g_timer.ev[(size_t)g_timer.calls * gdn::kNumStages * 2];
    ran = &g_timer.ran[(size_t)g_timer.calls];
    *ran = (1u << gdn::kNumStages) - 1;  // the launchers clear what does not run
    ++g_timer.calls;
  }
  hipError_t err = single
      ? gdn::launch_short_prefill(p, static_cast<hipStream_t>(stream), ev, ran)
      : gdn::launch_prefill(p, static_cast<hipStream_t>(stream), ev, ran);
  if (err != hipSuccess) {
    // a failed call's events may be unrecorded: the timing read skips it
    if (ran) *ran = 0;
    return fail(GDN_ERR_HIP, "HIP error: %s", hipGetErrorString(err));
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_decode(const gdn_desc* d, const void* q, const void* k,
                      const void* v, const void* a, const void* b,
                      const float* A_log, const float* dt_bias, const void* z,
                      const float* norm_w, float* state_cache,
                      int64_t num_slots, const int32_t* slot_idx, void* o,
                      void* stream) {
  g_err[0] = '\0';
  gdn_status st = check_desc(d);
  if (st != GDN_OK) return st;
  if (d->total_tokens != d->num_seqs)
    return fail(GDN_ERR_INVALID,
                "decode takes one token per request: total_tokens (%lld) must "
                "equal num_seqs (%d)", (long long)d->total_tokens, d->num_seqs);
  const int64_t B = d->num_seqs;
  if (num_slots < 1) return fail(GDN_ERR_INVALID, "num_slots must be >= 1");
  if (!slot_idx && num_slots < B)
    return fail(GDN_ERR_INVALID,
                "slot_idx is NULL, so request i uses slot i: num_slots (%lld) "
                "must be >= num_seqs (%lld)", (long long)num_slots, (long long)B);
  if ((z == nullptr) != (norm_w == nullptr))
    return fail(GDN_ERR_INVALID, "z and norm_w must both be given or both NULL");
  if (!A_log || !dt_bias) return fail(GDN_ERR_INVALID, "A_log/dt_bias is NULL");
  if (!q || !k || !v || !a || !b || !o || !state_cache)
    return fail(GDN_ERR_INVALID,
                "a tensor (q, k, v, a, b, o, state_cache) is NULL");
  size_t cache_elems;
  if (!mul_ok((size_t)num_slots, (size_t)d->hv * d->dv * d->dk, &cache_elems) ||
      cache_elems > (size_t)INT64_MAX / 4)
    return fail(GDN_ERR_UNSUPPORTED, "state cache size overflows");
  const void* vec_ptrs[] = {q, k, v, z, o, state_cache};
  const char* vec_names[] = {"q", "k", "v", "z", "o", "state_cache"};
  for (int i = 0; i < 6; ++i)
    if (vec_ptrs[i] && !aligned(vec_ptrs[i], 16))
      return fail(GDN_ERR_INVALID, "%s is not 16-byte aligned", vec_names[i]);
  const size_t esz = d->dtype == GDN_BF16 ? 2 : 4;
  if (!aligned(a, esz) || !aligned(b, esz) || !aligned(A_log, 4) ||
      !aligned(dt_bias, 4) || (norm_w && !aligned(norm_w, 4)) ||
      (slot_idx && !aligned(slot_idx, 4)))
    return fail(GDN_ERR_INVALID, "a, b, A_log, dt_bias, norm_w or slot_idx "
                                 "is misaligned for its element type");

  st = check_grid((uint64_t)B * (uint64_t)d->hv * 256, "decode");
  if (st != GDN_OK) return st;

  gdn::DecodeLaunch L;
  L.dtype = d->dtype == GDN_BF16 ? 1 : 0;
  L.B = d->num_seqs;
  L.Hk = d->hk;
  L.Hv = d->hv;
  L.scale = d->scale;
  L.l2_eps = d->qk_l2_eps;
  L.norm_eps = d->norm_eps;
  L.q = q;
  L.k = k;
  L.v = v;
  L.a = a;
  L.b = b;
  L.z = z;
  L.A_log = A_log;
  L.dt_bias = dt_bias;
  L.norm_w = norm_w;
  L.cache = state_cache;
  L.slots = slot_idx;
  L.num_slots = num_slots;
  L.o = o;
  hipError_t err = gdn::launch_decode(L, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(GDN_ERR_HIP, "HIP error: %s", hipGetErrorString(err));
  return GDN_OK;
}

gdn_status gdn_mfma_probe(int64_t iters, int32_t blocks, float* out, void* stream) {
  g_err[0] = '\0';
  if (iters < 1 || blocks < 1) return fail(GDN_ERR_INVALID, "iters and blocks must be >= 1");
  if (!out || !aligned(out, 4)) return fail(GDN_ERR_INVALID, "out is NULL or misaligned");
  hipError_t err = gdn::launch_mfma_probe(iters, blocks, out, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(GDN_ERR_HIP, "HIP error: %s", hipGetErrorString(err));
  return GDN_OK;
}

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK:
      return "GDN_OK";
    case GDN_ERR_INVALID:
      return "GDN_ERR_INVALID";
    case GDN_ERR_UNSUPPORTED:
      return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE:
      return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP:
      return "GDN_ERR_HIP";
  }
  return "GDN_ERR_UNKNOWN";
}

const char* gdn_last_error(void) { return g_err; }

int32_t gdn_version(void) { return 100; }

gdn_status gdn_stage_timing_enable(int32_t max_calls) {
  timer_release();
  if (max_calls < 0) return fail(GDN_ERR_INVALID, "max_calls < 0");
  if (max_calls == 0) return GDN_OK;
  const size_t n = (size_t)max_calls * gdn::kNumStages * 2;
  g_timer.ev.reserve(n);
  for (size_t i = 0; i < n; ++i) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      timer_release();
      return fail(GDN_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    g_timer.ev.push_back(e);
  }
  g_timer.ran.assign((size_t)max_calls, 0u);
  g_timer.max_calls = max_calls;
  g_timer.calls = 0;
  return GDN_OK;
}

int32_t gdn_stage_timing_read(double* ms_sum, const char** names, int32_t cap,
                              int32_t* calls) {
  if (calls) *calls = g_timer.calls;
  const int S = gdn::kNumStages;
  for (int s = 0; s < S && s < cap; ++s) {
    if (names) names[s] = kStageNames[s];
    if (ms_sum) ms_sum[s] = 0.0;
  }
  // only the stages each call ran were recorded; the others add nothing
  for (int c = 0; c < g_timer.calls; ++c) {
    hipEvent_t* e = &g_timer.ev[(size_t)c * S * 2];
    const unsigned ran = g_timer.ran[(size_t)c];
    for (int s = 0; s < S && s < cap; ++s) {
      if (!(ran & (1u << s))) continue;
      hipError_t err = hipEventSynchronize(e[2 * s + 1]);
      if (err != hipSuccess)
        return (int32_t)fail(GDN_ERR_HIP, "hipEventSynchronize: %s",
                             hipGetErrorString(err));
      float ms = 0.f;
      err = hipEventElapsedTime(&ms, e[2 * s], e[2 * s + 1]);
      if (err != hipSuccess)
        return (int32_t)fail(GDN_ERR_HIP, "hipEventElapsedTime: %s",
                             hipGetErrorString(err));
      if (ms_sum) ms_sum[s] += ms;
    }
  }
  return S;
}

gdn_status gdn_layer_desc_init(gdn_layer_desc* d, int32_t num_seqs,
                               int64_t total_tokens, int32_t hidden,
                               int32_t hk, int32_t hv, int32_t conv_width) {
  if (!d) return fail(GDN_ERR_INVALID, "layer desc is NULL");
  gdn_status st = gdn_desc_init(&d->op, num_seqs, total_tokens, hk, hv, 128,
                                128, GDN_BF16);
  if (st != GDN_OK) return st;
  d->hidden = hidden;
  d->conv_width = conv_width;
  d->conv_fused = 0;
  return GDN_OK;
}

size_t gdn_layer_workspace_size(const gdn_layer_desc* d) {
  if (check_layer(d) != GDN_OK) return 0;
  LayerLayout L;
  if (!plan_layer(d, &L)) return 0;
  return L.total;
}

gdn_status gdn_layer_prefill(const gdn_layer_desc* d, const void* x,
                             const void* W_in, const void* conv_w,
                             const float* A_log, const float* dt_bias,
                             const float* norm_w, const void* W_out,
                             const float* state_in, const void* conv_state_in,
                             const int32_t* cu_seqlens, void* out,
                             float* state_out, void* conv_state_out,
                             void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_err[0] = '\0';
  gdn_status st = check_layer(d);
  if (st != GDN_OK) return st;
  const gdn_desc& op = d->op;
  if (!cu_seqlens && op.num_seqs != 1)
    return fail(GDN_ERR_INVALID, "cu_seqlens is NULL but num_seqs = %d",
                op.num_seqs);
  if (!A_log || !dt_bias || !norm_w)
    return fail(GDN_ERR_INVALID, "A_log, dt_bias and norm_w are required");
  if (op.total_tokens > 0 && (!x || !out))
    return fail(GDN_ERR_INVALID, "x or out is NULL");
  if (!W_in || !conv_w || !W_out)
    return fail(GDN_ERR_INVALID, "a weight (W_in, conv_w, W_out) is NULL");
  const void* p16[] = {x, W_in, W_out, out, state_in, state_out, conv_state_in,
                       conv_state_out};
  const char* n16[] = {"x", "W_in", "W_out", "out", "state_in", "state_out",
                       "conv_state_in", "conv_state_out"};
  for (int i = 0; i < 8; ++i)
    if (p16[i] && !aligned(p16[i], 16))
      return fail(GDN_ERR_INVALID, "%s is not 16-byte aligned", n16[i]);
  if (!aligned(conv_w, 16))
    return fail(GDN_ERR_INVALID, "conv_w is not 16-byte aligned");
  LayerLayout L;
  if (!plan_layer(d, &L))
    return fail(GDN_ERR_UNSUPPORTED, "workspace size overflows");
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                L.total, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256))
    return fail(GDN_ERR_INVALID, "workspace is not 256-byte aligned");
  const int64_t T = op.total_tokens;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto bf = [&](size_t off) { return reinterpret_cast<__bf16*>(ws + off); };

  if (conv_state_in && conv_state_out && conv_state_in != conv_state_out) {
    const size_t bytes =
        (size_t)op.num_seqs * (d->conv_width - 1) * (size_t)(2 * L.Wq + L.Wv) * 2;
    const char* i0 = static_cast<const char*>(conv_state_in);
    const char* o0 = static_cast<const char*>(conv_state_out);
    if (bytes > 0 && i0 < o0 + bytes && o0 < i0 + bytes)
      return fail(GDN_ERR_INVALID, "conv_state_in and conv_state_out partially overlap");
  }
  // 2. causal conv + SiLU over q|k|v (and the new conv history)
  gdn::ConvArgs c{};
  c.x = bf(L.P);
  c.ldx = 2 * L.Wq + L.Wv;
  c.w = static_cast<const __bf16*>(conv_w);
  c.W = d->conv_width;
  c.T = T;
  c.C = (int)(2 * L.Wq + L.Wv);
  c.cu = cu_seqlens;
  c.N = op.num_seqs;
  c.dst[0] = bf(L.q);
  c.dld[0] = L.Wq;
  c.dcol0[0] = 0;
  c.dst[1] = bf(L.k);
  c.dld[1] = L.Wq;
  c.dcol0[1] = (int)L.Wq;
  c.dst[2] = bf(L.v);
  c.dld[2] = L.Wv;
  c.dcol0[2] = (int)(2 * L.Wq);
  c.hin = static_cast<const __bf16*>(conv_state_in);
  c.hout = static_cast<__bf16*>(conv_state_out);
  if (T > 0) {
    // 1. packed input projection, its columns split into P (q|k|v), z, b, a
    gdn::GemmArgs g{};
    g.A = static_cast<const __bf16*>(x);
    g.B = static_cast<const __bf16*>(W_in);
    g.lda = d->hidden;
    g.ldb = d->hidden;
    g.M = T;
    g.N = L.Wp;
    g.K = d->hidden;
    g.nseg = 4;
    g.col0[0] = 0;
    g.ptr[0] = bf(L.P);
    g.ld[0] = 2 * L.Wq + L.Wv;
    g.col0[1] = 2 * L.Wq + L.Wv;
    g.ptr[1] = bf(L.z);
    g.ld[1] = L.Wv;
    g.col0[2] = 2 * L.Wq + 2 * L.Wv;
    g.ptr[2] = bf(L.b);
    g.ld[2] = op.hv;
    g.col0[3] = 2 * L.Wq + 2 * L.Wv + op.hv;
    g.ptr[3] = bf(L.a);
    g.ld[3] = op.hv;
    hipError_t err = gdn::launch_gemm(g, hs);
    if (err != hipSuccess)
      return fail(GDN_ERR_HIP, "in_proj: %s", hipGetErrorString(err));
  }
  // 2-3. the conv, then the gated delta rule with the gated norm (which
  // also carries the state through when T == 0).  With conv_fused set, when
  // the chunked kernels run, the conv is applied by their first kernel to
  // the rows it stages, and only the new conv history runs on its own,
  // after it (conv_state_out may be conv_state_in).
  const bool fused = d->conv_fused && T > 0 && !short_applies(&op);
  if (fused) {
    gdn::PrepConv pc;
    pc.x = bf(L.P);
    pc.ldx = 2 * L.Wq + L.Wv;
    pc.w = conv_w;
    pc.hin = conv_state_in;
    pc.W = d->conv_width;
    pc.C = (int)(2 * L.Wq + L.Wv);
    g_err[0] = '\0';
    st = prefill_impl(&op, bf(L.q), bf(L.k), bf(L.v), bf(L.a), bf(L.b), A_log, dt_bias,
                      bf(L.z), norm_w, state_in, cu_seqlens, bf(L.y), state_out, ws + L.op,
                      workspace_bytes - L.op, stream, &pc);
    if (st != GDN_OK) return st;
    if (conv_state_out) {
      hipError_t err = gdn::launch_conv_history(c, hs);
      if (err != hipSuccess)
        return fail(GDN_ERR_HIP, "conv history: %s", hipGetErrorString(err));
    }
  } else {
    if (T > 0 || conv_state_out) {
      // with no tokens this only carries the conv history through
      hipError_t err = gdn::launch_conv_silu(c, hs);
      if (err != hipSuccess)
        return fail(GDN_ERR_HIP, "conv: %s", hipGetErrorString(err));
    }
    st = gdn_prefill(&op, bf(L.q), bf(L.k), bf(L.v), bf(L.a), bf(L.b), A_log,
                     dt_bias, T > 0 ? bf(L.z) : nullptr, norm_w, state_in,
                     cu_seqlens, bf(L.y), state_out, ws + L.op,
                     workspace_bytes - L.op, stream);
    if (st != GDN_OK) return st;
  }
  if (T > 0) {
    // 4. output projection
    gdn::GemmArgs g{};
    g.A = bf(L.y);
    g.B = static_cast<const __bf16*>(W_out);
    g.lda = L.Wv;
    g.ldb = L.Wv;
    g.M = T;
    g.N = d->hidden;
    g.K = L.Wv;
    g.nseg = 1;
    g.col0[0] = 0;
    g.ptr[0] = out;
    g.ld[0] = d->hidden;
    hipError_t err = gdn::launch_gemm(g, hs);
    if (err != hipSuccess)
      return fail(GDN_ERR_HIP, "out_proj: %s", hipGetErrorString(err));
  }
  return GDN_OK;
}

gdn_status gdn_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A,
                         int64_t lda, const void* B, int64_t ldb, void* C,
                         int64_t ldc, void* stream) {
  g_err[0] = '\0';
  if (M < 0 || N < 0 || K < 0) return fail(GDN_ERR_INVALID, "negative size");
  if (M == 0 || N == 0) return GDN_OK;
  if (K % 32 != 0 || K == 0)
    return fail(GDN_ERR_UNSUPPORTED, "K (%lld) must be a positive multiple of 32",
                (long long)K);
  if (!A || !B || !C) return fail(GDN_ERR_INVALID, "A, B or C is NULL");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 2))
    return fail(GDN_ERR_INVALID, "A/B not 16-byte aligned or C misaligned");
  if (lda < K || ldb < K || ldc < N || lda % 8 || ldb % 8)
    return fail(GDN_ERR_INVALID, "bad leading dimensions");
  gdn::GemmArgs g{};
  g.A = static_cast<const __bf16*>(A);
  g.B = static_cast<const __bf16*>(B);
  g.lda = lda;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.nseg = 1;
  g.col0[0] = 0;
  g.ptr[0] = C;
  g.ld[0] = ldc;
  hipError_t err = gdn::launch_gemm(g, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(GDN_ERR_HIP, "HIP error: %s", hipGetErrorString(err));
  return GDN_OK;
}

gdn_status gdn_conv_silu_bf16(int64_t T, int32_t C, int32_t W, const void* x,
                              int64_t ldx, const void* w, const void* hist_in,
                              const int32_t* cu_seqlens, int32_t num_seqs,
                              void* y, void* hist_out, void* stream) {
  g_err[0] = '\0';
  if (T < 0 || C < 0) return fail(GDN_ERR_INVALID, "negative size");
  if (W < 1 || W > 4) return fail(GDN_ERR_UNSUPPORTED, "W must be in 1..4");
  if (C % 8 != 0 || ldx % 8 != 0 || ldx < C)
    return fail(GDN_ERR_UNSUPPORTED, "C and ldx must be multiples of 8, ldx >= C");
  if (!cu_seqlens && num_seqs != 1)
    return fail(GDN_ERR_INVALID, "cu_seqlens is NULL but num_seqs = %d", num_seqs);
  if (num_seqs < 1) return fail(GDN_ERR_INVALID, "num_seqs must be >= 1");
  if (C == 0 || (T == 0 && !hist_out)) return GDN_OK;
  if (T > 0 && (!x || !w || !y)) return fail(GDN_ERR_INVALID, "x, w or y is NULL");
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)) || (w && !aligned(w, 16)) ||
      (hist_in && !aligned(hist_in, 16)) || (hist_out && !aligned(hist_out, 16)))
    return fail(GDN_ERR_INVALID, "x, w, y, hist_in or hist_out is not 16-byte aligned");
  if (hist_in && hist_out && hist_in != hist_out) {
    const size_t bytes = (size_t)num_seqs * (W - 1) * (size_t)C * 2;
    const char* i0 = static_cast<const char*>(hist_in);
    const char* o0 = static_cast<const char*>(hist_out);
    if (bytes > 0 && i0 < o0 + bytes && o0 < i0 + bytes)
      return fail(GDN_ERR_INVALID, "hist_in and hist_out partially overlap");
  }
  gdn::ConvArgs c{};
  c.x = static_cast<const __bf16*>(x);
  c.ldx = ldx;
  c.w = static_cast<const __bf16*>(w);
  c.W = W;
  c.T = T;
  c.C = C;
  c.cu = cu_seqlens;
  c.N = num_seqs;
  for (int dd = 0; dd < 3; ++dd) {
    c.dst[dd] = static_cast<__bf16*>(y);
    c.dld[dd] = C;
    c.dcol0[dd] = dd == 0 ? 0 : C;  // one destination
  }
  c.hin = static_cast<const __bf16*>(hist_in);
  c.hout = static_cast<__bf16*>(hist_out);
  hipError_t err = gdn::launch_conv_silu(c, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(GDN_ERR_HIP, "HIP error: %s", hipGetErrorString(err));
  return GDN_OK;
}

}  // extern "C"
