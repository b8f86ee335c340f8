/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule prefill library
 * (libgdn.so).  Plain C: no C++ types, no exceptions, no torch types.
 *
 * The operation (sources, by page title and section):
 *   "Add opt-in fused Qwen3.5 inference kernels" (JevAny PR #29), Summary:
 *     the Gated DeltaNet chunked kernel applies the decay gate built from
 *     A_log and dt_bias, a sigmoid beta, q/k L2 normalisation and grouped
 *     value heads; a fused gated RMSNorm follows it.  The DeltaNet fast path
 *     there refuses packed-sequence metadata; this library accepts it.
 *   "feat(qwen35): add SM120 FlashInfer GDN prefill candidate" (pegainfer
 *     PR #862), Summary / Correctness / Performance: the linear-attention
 *     prefill operation with backend-owned scratch, chunked vs unchunked
 *     prefill with carried state, HKV/HVK state layouts and alias handling,
 *     CUDA-graph integration, explicit handling of unsupported shapes.
 *
 * Per token t of a sequence and value head h (key head kh = h / (hv/hk)):
 *   g_t   = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 *   beta  = sigmoid(b[t,h])
 *   qn    = scale * q[t,kh] / sqrt(|q[t,kh]|^2 + qk_l2_eps)
 *   kn    =         k[t,kh] / sqrt(|k[t,kh]|^2 + qk_l2_eps)
 *   S_t   = exp(g_t) S_{t-1} (I - beta kn kn^T) + beta v[t,h] kn^T
 *   o_t   = S_t qn
 *   y_t   = o_t / sqrt(mean(o_t^2) + norm_eps) * norm_w * silu(z[t,h])
 *           (only when z and norm_w are given; y replaces o)
 * S is a dv x dk fp32 matrix per (sequence, value head).
 *
 * Conventions for every call below:
 *   - Tensors are caller-owned, dense, row-major device pointers, aligned to
 *     16 bytes.  The library never allocates or frees device memory on the
 *     call path; scratch comes from the caller's workspace.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  There is no host synchronisation and no host read of device
 *     data, so a call can be captured into a HIP graph.
 *   - The return value is a gdn_status.  Arguments are validated on the host
 *     before anything is launched; on error nothing is launched and
 *     gdn_last_error() describes the problem.  Unsupported shapes return
 *     GDN_ERR_UNSUPPORTED; there is no silent fallback.  So do calls whose
 *     largest kernel grid would exceed 2^32 - 1 work-items (the dispatch
 *     packet's limit), e.g. a decode batch of 2^20 requests over 32 value
 *     heads; such a call must be split by the caller.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID = -1,     /* null / inconsistent / misaligned arguments */
  GDN_ERR_UNSUPPORTED = -2, /* valid, but not implemented on the GPU path */
  GDN_ERR_WORKSPACE = -3,   /* workspace missing or too small */
  GDN_ERR_HIP = -4          /* a HIP runtime call or launch failed */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Shape and options of one prefill call. */
typedef struct {
  int32_t num_seqs;     /* N >= 1; must be 1 when cu_seqlens is NULL */
  int64_t total_tokens; /* T_tot >= 0: rows of q, k, v, a, b, z, o */
  int32_t hq, hk, hv;   /* hq == hk; hv % hk == 0 (grouped value heads) */
  int32_t dk, dv;       /* head dims; the GPU path implements 128, 128 */
  int32_t dtype;        /* gdn_dtype of q, k, v, a, b, z and o */
  float scale;          /* multiplies the L2-normalised q (usual: dk^-1/2) */
  float qk_l2_eps;      /* epsilon inside the q/k L2 norms (usual: 1e-6) */
  float norm_eps;       /* epsilon of the gated RMSNorm (usual: 1e-6) */
  int32_t short_tokens; /* L >= 0 of gdn_prefill's single-kernel bound below
                           (usual: 8; 0 sends every call to the chunked
                           kernels).  Part of the call's description, so
                           which kernels compute a call depends on nothing
                           but its arguments. */
  int32_t chain_segments; /* how the chunk-to-chunk state chain runs: 0 (usual)
                           lets the library choose; 1 runs it as one pass
                           per sequence; G >= 2 splits a single sequence
                           (num_seqs == 1) into G segments scanned in
                           parallel (GDN_ERR_UNSUPPORTED for num_seqs > 1).
                           See gdn_prefill. */
} gdn_desc;

/* Fills `d` with the usual defaults for the given shape (scale = dk^-1/2,
 * both epsilons 1e-6, short_tokens 8, chain_segments 0).  Returns
 * GDN_ERR_INVALID if d is NULL. */
gdn_status gdn_desc_init(gdn_desc* d, int32_t num_seqs, int64_t total_tokens,
                         int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                         int32_t dtype);

/* Bytes of device workspace gdn_prefill needs for `d` (0 if d is invalid).
 * Pure host computation.  The amount depends on total_tokens, num_seqs,
 * hk, hv and dtype only. */
size_t gdn_prefill_workspace_size(const gdn_desc* d);

/*
 * Gated delta rule prefill over a packed batch of sequences.
 *
 *   q         [T_tot, hq, dk]   dtype
 *   k         [T_tot, hk, dk]   dtype
 *   v         [T_tot, hv, dv]   dtype
 *   a, b      [T_tot, hv]       dtype  (gate and beta pre-activations)
 *   A_log     [hv]              fp32
 *   dt_bias   [hv]              fp32
 *   z         [T_tot, hv, dv]   dtype, or NULL  } both NULL: no gated norm,
 *   norm_w    [dv]              fp32,  or NULL  } o receives S_t qn
 *             (when T_tot == 0, z may be NULL whatever norm_w is)
 *   state_in  [N, hv, dv, dk]   fp32, or NULL (zeros).  Layout is "HVK":
 *             state_in[n][h][i][j] = S[i][j] of the recurrence above.
 *   cu_seqlens[N + 1]           int32 device array, or NULL (one sequence
 *             of T_tot tokens).  cu_seqlens[0] = 0, non-decreasing,
 *             cu_seqlens[N] = T_tot.  Zero-length sequences are allowed (their
 *             state passes through).  It is read on the device only; values
 *             outside [0, T_tot] are clamped, which keeps every access in
 *             bounds but makes the result unspecified.
 *   o         [T_tot, hv, dv]   dtype, out (y when the gated norm is on).
 *             Rounded to dtype with round-to-nearest-even.
 *   state_out [N, hv, dv, dk]   fp32, out, or NULL (not written).  May be the
 *             same pointer as state_in (in place); partial overlap is
 *             undefined.
 *   workspace, workspace_bytes: device scratch of at least
 *             gdn_prefill_workspace_size(d) bytes, 256-byte aligned.  Its
 *             contents on entry do not matter; it is not read after the
 *             call's kernels finish.  One workspace must not be shared by
 *             calls that may run concurrently.
 *   stream    hipStream_t or NULL.
 *
 * Precision: fp32 state, gates and accumulation; for GDN_BF16 the matrix
 * products take bf16 operands (MFMA), for GDN_F32 fp32 operands.
 *
 * A call of at most L + 2 (N - 1) tokens in all (N = num_seqs, L =
 * d->short_tokens) runs the recurrence token by token in fp32 in a single
 * kernel, which has far less fixed cost than the chunked
 * kernels; its results differ from theirs only by rounding.  It does not
 * touch the workspace, but the workspace argument is checked the same way.
 *
 * The chunked form carries the state from chunk to chunk in order, which
 * for one long sequence over few value heads keeps most of the GPU idle.
 * There, the chain may run as a sequence-parallel scan (d->chain_segments):
 * each chunk is an affine map of the state, so G segments of the sequence
 * are mapped in parallel (from a zero state, and from the identity with v
 * taken as zero), their start states composed in order, and the segments
 * run again in parallel from those states.  With the usual 0, the library
 * scans a single sequence when the per-segment work still fits the GPU
 * (value heads x 8 column blocks x (2G - 3) blocks in flight) and every
 * segment keeps at least 8 chunks; results differ from one pass only by
 * rounding.
 */
gdn_status gdn_prefill(const gdn_desc* d, const void* q, const void* k,
                       const void* v, const void* a, const void* b,
                       const float* A_log, const float* dt_bias, const void* z,
                       const float* norm_w, const float* state_in,
                       const int32_t* cu_seqlens, void* o, float* state_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments and kernels, with no workspace argument.
 * The scratch the kernels use lives in a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES (96 MiB) per GPU, held from the library's
 * first use on that GPU until the process ends; the call itself allocates
 * nothing.  A call whose gdn_prefill_workspace_size(d) exceeds it returns
 * GDN_ERR_WORKSPACE (at the Qwen3.5-4B geometry, hk 16 / hv 32 bf16, that
 * holds up to 2944 tokens in one sequence).  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (other
 * streams, other threads) race, and must be ordered by the caller.  The
 * array's contents between calls do not matter.  The array used is the
 * current device's (hipGetDevice), so `stream` must belong to that device
 * (GDN_ERR_INVALID otherwise).
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
gdn_status gdn_prefill_noalloc(const gdn_desc* d, const void* q, const void* k,
                               const void* v, const void* a, const void* b,
                               const float* A_log, const float* dt_bias,
                               const void* z, const float* norm_w,
                               const float* state_in, const int32_t* cu_seqlens,
                               void* o, float* state_out, void* stream);

/*
 * One decode step: a single new token for each of B requests, continuing
 * the sequence whose state is held in a slot of a state cache.  The step is
 * the recurrence above for one token (the decay, the delta write, o = S qn,
 * then the gated norm), as the prefill of a one-token sequence from that
 * state would compute it; the cache in slots ("mamba slots" in "[Perf] Pack
 * the Qwen3.5 GDN input projection on CUDA, including from the dense
 * wrapper" (sglang PR #42126), Accuracy Tests) is what a serving loop keeps
 * between steps.
 *
 *   d            num_seqs = total_tokens = B (one token per request);
 *                hq, hk, hv, dk, dv, dtype, scale, eps as gdn_prefill
 *   q, k         [B, hk, dk]  dtype
 *   v            [B, hv, dv]  dtype
 *   a, b         [B, hv]      dtype
 *   A_log, dt_bias [hv] fp32
 *   z, norm_w    as gdn_prefill (both NULL: o receives S qn)
 *   state_cache  [num_slots, hv, dv, dk] fp32, HVK as state_in; read and
 *                updated in place for the slots the batch names
 *   num_slots    >= 1
 *   slot_idx     int32 device array [B], or NULL (request i uses slot i;
 *                then num_slots >= B).  A value outside [0, num_slots)
 *                marks a padding entry: its o row is written as zeros and
 *                no slot is touched.  Live entries must name distinct
 *                slots; two requests on one slot race.
 *   o            [B, hv, dv]  dtype, out
 *   stream       hipStream_t or NULL
 *
 * No workspace.  Precision: everything in fp32 (vector ALU
 * matrix-vector products), o rounded to dtype with round-to-nearest-even.
 */
gdn_status gdn_decode(const gdn_desc* d, const void* q, const void* k,
                      const void* v, const void* a, const void* b,
                      const float* A_log, const float* dt_bias, const void* z,
                      const float* norm_w, float* state_cache,
                      int64_t num_slots, const int32_t* slot_idx, void* o,
                      void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* gdn_status_string(gdn_status s);

/* Detail of the last error returned on the calling thread (static
 * thread-local buffer; "" if none). */
const char* gdn_last_error(void);

/* Library version, as 10000 * major + 100 * minor + patch. */
int32_t gdn_version(void);

/*
 * Per-kernel timing of gdn_prefill, for measurement tools.  While enabled on
 * a thread, each gdn_prefill call on that thread attaches a start and an end
 * HIP event to each of its kernel dispatches (on the call's stream;
 * hipExtLaunchKernel), so each pair spans that kernel's execution alone, for
 * up to `max_calls` calls.  Timing changes no routing: a timed call runs the
 * same kernels as an untimed one.  gdn_stage_timing_read synchronises on
 * those events and returns, per stage, the summed elapsed milliseconds and
 * the number of calls timed; a stage a call does not run counts 0 for it.
 * Stage names: "prep", "chain", "out" (the chunked kernels) and "short"
 * (the single-kernel form).
 *   gdn_stage_timing_enable(max_calls > 0) creates the events (host-side
 *   HIP objects, no device memory) and resets the sums; max_calls == 0
 *   disables timing and releases them.
 *   gdn_stage_timing_read fills up to `cap` entries of ms_sum and names
 *   (either may be NULL) and returns the number of stages, or a negative
 *   gdn_status on error; *calls receives the number of timed calls.
 */
gdn_status gdn_stage_timing_enable(int32_t max_calls);
int32_t gdn_stage_timing_read(double* ms_sum, const char** names, int32_t cap,
                              int32_t* calls);

/*
 * Measurement only: a probe of the bf16 MFMA rate the device sustains, for
 * reporting rooflines against a measured peak beside the datasheet one.
 * `blocks` blocks of 256 threads; every wave runs `iters` rounds of eight
 * independent 16x16x32 bf16 MFMAs on register operands (2 * 16 * 16 * 32 *
 * 8 * iters FLOP per wave) and writes one float per thread to out
 * (blocks * 256 floats, device memory).  Time it with events on `stream`.
 */
gdn_status gdn_mfma_probe(int64_t iters, int32_t blocks, float* out, void* stream);

/*
 * Full Gated DeltaNet layer (prefill) around gdn_prefill.  The layer's four
 * input projections run as one GEMM ("Add opt-in fused Qwen3.5 inference
 * kernels" (JevAny PR #29), Summary), whose packed output is 12,352 wide at
 * the Qwen3.5-4B geometry ("[Perf] Pack the Qwen3.5 GDN input projection on
 * CUDA, including from the dense wrapper" (sglang PR #42126),
 * Modifications); a depthwise causal conv1d + SiLU runs over its q|k|v
 * channels before the gated delta rule.  With T = total_tokens,
 * Wq = hk*dk, Wv = hv*dv:
 *   P     = x W_in^T                [T, 2Wq + 2Wv + 2hv], columns in the order
 *                                    q (Wq) | k (Wq) | v (Wv) | z (Wv) | b (hv)
 *                                    | a (hv)
 *   c     = silu(conv(P[:, 0:2Wq+Wv]))  c[t][ch] = silu(sum_{j<W}
 *           conv_w[ch][j] * P[t - W + 1 + j][ch]), where the W - 1 rows
 *           before each sequence's first token are its conv history
 *           (conv_state_in below; zeros when that is NULL)
 *   y     = gdn_prefill(q = c[:, 0:Wq], k = c[:, Wq:2Wq], v = c[:, 2Wq:],
 *                       a, b, z, norm_w, state)   (gated norm on)
 *   out   = y W_out^T               [T, hidden]
 * Intermediates (P, c, y) are rounded to bf16 as they are stored.
 */
typedef struct {
  gdn_desc op;        /* the prefill; dtype must be GDN_BF16, dk = dv = 128 */
  int32_t hidden;     /* model width: columns of x and of out (multiple of 32) */
  int32_t conv_width; /* causal conv width W, 1..4 */
  int32_t conv_fused; /* 0 (usual): the conv runs as a kernel of its own
                         before the prefill; 1: when the prefill runs its
                         chunked kernels, the first of them applies the conv
                         to the rows it stages and writes the post-conv rows
                         the others read (the same results, bit for bit;
                         slower at the Qwen3.5-4B geometry: its first kernel
                         then holds the conv's tap rows in registers at
                         half the occupancy) */
} gdn_layer_desc;

/* Defaults as gdn_desc_init (bf16, dk = dv = 128) plus hidden and the conv
 * width; conv_fused 0.  Returns GDN_ERR_INVALID if d is NULL. */
gdn_status gdn_layer_desc_init(gdn_layer_desc* d, int32_t num_seqs,
                               int64_t total_tokens, int32_t hidden,
                               int32_t hk, int32_t hv, int32_t conv_width);

/* Bytes of device workspace gdn_layer_prefill needs (0 if d is invalid). */
size_t gdn_layer_workspace_size(const gdn_layer_desc* d);

/*
 *   x         [T, hidden]                  bf16
 *   W_in      [2Wq + 2Wv + 2hv, hidden]    bf16 ([out, in] layout)
 *   conv_w    [2Wq + Wv, W]                bf16
 *   A_log, dt_bias [hv] fp32; norm_w [dv] fp32 (all required)
 *   W_out     [hidden, Wv]                 bf16 ([out, in] layout)
 *   state_in, cu_seqlens, state_out: as gdn_prefill
 *   conv_state_in  [N, W - 1, 2Wq + Wv]    bf16, or NULL (zeros): per
 *             sequence, the W - 1 conv input rows (pre-conv q | k | v, oldest
 *             first) that precede its first token -- the history a previous
 *             call on the same sequences returned
 *   out       [T, hidden]                  bf16, out
 *   conv_state_out [N, W - 1, 2Wq + Wv]    bf16, out, or NULL (not
 *             written): each sequence's last W - 1 conv input rows, taken
 *             from conv_state_in where the sequence is shorter.  May be the
 *             same pointer as conv_state_in; partial overlap is rejected.
 *   workspace: gdn_layer_workspace_size(d) bytes, 256-byte aligned
 * With both states carried, one call over tokens [0, T) gives the same
 * result as two calls over [0, T1) and [T1, T) (the conv history and the
 * recurrent state are all that connect them).  Same conventions as
 * gdn_prefill (asynchronous, validated on the host, no allocation).  out
 * must not overlap any input.
 */
gdn_status gdn_layer_prefill(const gdn_layer_desc* d, const void* x,
                             const void* W_in, const void* conv_w,
                             const float* A_log, const float* dt_bias,
                             const float* norm_w, const void* W_out,
                             const float* state_in, const void* conv_state_in,
                             const int32_t* cu_seqlens, void* out,
                             float* state_out, void* conv_state_out,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * The layer's projection GEMM on its own: C[M][N] = A[M][K] B[N][K]^T with
 * bf16 A, B, C (row strides lda, ldb, ldc in elements) and fp32
 * accumulation, C rounded to nearest even.  K must be a multiple of 32;
 * pointers 16-byte aligned, lda and ldb multiples of 8.
 */
gdn_status gdn_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A,
                         int64_t lda, const void* B, int64_t ldb, void* C,
                         int64_t ldc, void* stream);

/*
 * The layer's conv on its own: y[t][c] = silu(sum_{j<W} w[c][j] *
 * x[t - W + 1 + j][c]), where a row before the first token s of sequence n
 * is its history, x[s - d] = hist_in[n][W - 1 - d] (d = 1 .. W - 1), or
 * zero when hist_in is NULL.  x [T][C] with row stride ldx, w [C][W], y
 * dense [T][C], hist_in / hist_out [N][W - 1][C], all bf16 (C a multiple
 * of 8, ldx a multiple of 8, W in 1..4; every pointer 16-byte aligned).
 * hist_out (or NULL) receives each sequence's last W - 1 rows of x, taken
 * from hist_in where the sequence is shorter; it may be hist_in.
 * cu_seqlens as gdn_prefill (NULL: one sequence; num_seqs its entry count
 * minus one).
 */
gdn_status gdn_conv_silu_bf16(int64_t T, int32_t C, int32_t W, const void* x,
                              int64_t ldx, const void* w, const void* hist_in,
                              const int32_t* cu_seqlens, int32_t num_seqs,
                              void* y, void* hist_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
