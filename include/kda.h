/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * The operator (readings of the pages; the page title and section are cited
 * at each call):
 *   per sequence and head, with fp32 state S in R^{dk x dv} starting at h0
 *   (or 0), for every token t
 *       S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *       o_t = scale * S_t^T q_t
 *   i.e. the delta-rule recurrence with a per-channel decay gate
 *   ("Pure KDA 300M on Primus" guide, Overview; openkimi README, What is
 *   implemented, and its FlashQLA paragraph: KDA's decay is channel-wise),
 *   computed chunk by chunk (chunks of 64 tokens, in-chunk WY/UT form) with
 *   optional document offsets that reset the state at every document start
 *   (torchtitan PR #4347 "[kimi k3] Support sample packing in KDA",
 *   Verification).
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer, contiguous, 16-byte aligned,
 *     row-major in the layout given at the call.  Token-major layouts
 *     [B,T,H,d] follow the [B,T,D] activations of the Primus guide
 *     (Troubleshooting: keep [B,T,D], call .contiguous()).
 *   - The caller owns every buffer, including the workspace sized by the
 *     *_workspace queries.  The library never allocates, frees or
 *     synchronizes, and never reads device memory on the host.
 *   - All work is enqueued on `stream` (a hipStream_t; 0 = the null stream).
 *   - Every call declared `int` returns a kda_status value (the enum below;
 *     `int` keeps the ABI's return type fixed-width across compilers).
 *   - Arguments are checked from the descriptor and the pointer values only.
 *     On any error the call returns before launching anything and leaves all
 *     outputs untouched; kda_last_error() then describes it (thread-local).
 *   - Results are deterministic run to run (no floating-point atomics).
 *   - No output may alias an input, except the in-place state of kda_step.
 *   - Empty inputs (T = 0, or rows = 0 for the gated norm) are valid: the
 *     per-token (per-row) arrays may then be null; states pass through
 *     (hT = h0, dh0 = dhT) and parameter gradients are written as zeros.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layout-compatible with hipStream_t, so this header needs no HIP include. */
typedef struct ihipStream_t* kda_stream_t;

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID = 1,     /* bad shape, null/misaligned pointer, bad flag */
    KDA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. dk, dv pair) */
    KDA_ERR_WORKSPACE = 3,   /* workspace null or too small */
    KDA_ERR_HIP = 4          /* a HIP launch failed */
} kda_status;

typedef enum kda_dtype { KDA_BF16 = 0, KDA_FP32 = 1 } kda_dtype;

/* Optional fused preparation (openkimi README, What is implemented: fused
 * Q/K norm, decay gate and beta; Primus guide, Overview: decay gate with
 * learnable A_log and dt_bias through softplus).  With a flag set, the
 * corresponding argument holds the RAW input and gradients are returned with
 * respect to that raw input.
 *   KDA_F_QK_L2NORM      q, k are normalised per token and head in-kernel:
 *                        x^ = x * (sum x^2 + 1e-6)^(-1/2)
 *   KDA_F_GATE_IN_KERNEL the `g` argument holds f; the log-decay is
 *                        g = -exp(A_log[h]) * softplus(f + dt_bias[h][c]),
 *                        softplus(x) = log1p(exp(x)) (x <= 20), x (x > 20)
 *   KDA_F_BETA_LOGITS    the `beta` argument holds logits b; beta = sigmoid(b) */
enum {
    KDA_F_QK_L2NORM = 1u << 0,
    KDA_F_GATE_IN_KERNEL = 1u << 1,
    KDA_F_BETA_LOGITS = 1u << 2,
    KDA_F_SAVE_FOR_BWD = 1u << 3,
    KDA_F_FWD_SAVED = 1u << 4,
    KDA_F_DH0_ONLY = 1u << 5
};
/* Saving the forward for the backward (the usual training pattern):
 *   KDA_F_SAVE_FOR_BWD  (kda_fwd) also keep, in the workspace, the per-chunk
 *                       quantities the backward needs (the UT inverse, the
 *                       state entering every chunk, v_new); the workspace must
 *                       then hold kda_bwd_workspace(desc) bytes.
 *   KDA_F_FWD_SAVED     (kda_bwd) read them from `ws` instead of recomputing
 *                       the forward.  `ws` must be the workspace of a kda_fwd
 *                       call with KDA_F_SAVE_FOR_BWD on the same descriptor
 *                       (other flags equal), inputs and varlen tables, with
 *                       nothing written to it in between.  The results are
 *                       identical to a backward that recomputes.
 *                       (kda_fwd) the intra-chunk quantities of these inputs
 *                       are in `ws` already (from a kda_fwd with
 *                       KDA_F_SAVE_FOR_BWD): only the state pass runs, from
 *                       this call's h0 (with KDA_F_SAVE_FOR_BWD too it keeps
 *                       the new states for the backward).
 *                       (kda_segment_maps) read the chunks' transitions from
 *                       such a `ws` instead of forming them.
 *   KDA_F_DH0_ONLY      (kda_bwd) run the reverse state pass alone: only dh0
 *                       (required) is written; dq, dk, dv, dg, dbeta, dA_log
 *                       and ddt_bias may be null and are left untouched. */

/* Problem descriptor.
 *   B      rows (B == 1 when packed)
 *   T      tokens per row (dense) or total tokens of the packed row; T >= 0
 *   H      heads (one head count for q, k and v: Primus guide, Overview)
 *   dk,dv  head dims; supported pairs (32,64), (64,64), (128,128)
 *   N      sequences: == B when dense, number of documents when packed
 *   chunk  chunk length, must be 64
 *   dtype      element type of q, k, v (and d_o in kda_bwd)
 *   out_dtype  element type of o (kda_fwd) and dq, dk, dv (kda_bwd); bf16
 *              outputs are the round-to-nearest-even of the fp32 result
 *   scale  output scale (the caller passes dk^-0.5 for the usual choice)
 *   flags  KDA_F_* above */
typedef struct kda_desc {
    int32_t B, T, H, dk, dv, N, chunk;
    kda_dtype dtype;
    kda_dtype out_dtype;
    float scale;
    uint32_t flags;
} kda_desc;

/* Host-only upper bound on the number of chunks that N documents totalling T
 * tokens can have: floor((T + N*(chunk-1)) / chunk).  Returns -1 on bad
 * arguments.  Size chunk_indices for kda_plan_varlen with it.
 * (torchtitan PR #4347, Performance: the per-batch offset tables are built
 * without a device-to-host copy; this bound sizes them, and the grid of every
 * packed call, from host integers alone -- surplus workgroups exit.) */
int32_t kda_max_chunks(int32_t T, int32_t N, int32_t chunk);

/* Per-document chunk metadata for a packed row (torchtitan PR #4347: the
 * offsets are turned into chunk tables once per batch and shared by every
 * layer, forward and backward).  Device inputs/outputs:
 *   cu_seqlens     int32 [N+1], cu[0] = 0, non-decreasing, cu[N] = T
 *                  (a precondition, not checked on the device path; see
 *                  kda_check_cu_seqlens)
 *   chunk_indices  int32 [kda_max_chunks(T,N,chunk)][2], rows (doc n, chunk i)
 *                  for n ascending and i = 0..ceil(L_n/chunk)-1; rows past the
 *                  real count are filled with (-1,-1)
 *   chunk_offsets  int32 [N+1], exclusive prefix sum of ceil(L_n/chunk)
 * Chunk (n,i) covers tokens [cu[n] + i*chunk, min(cu[n] + (i+1)*chunk, cu[n+1])):
 * chunks restart at each document, so a packed document is tiled exactly as
 * it is when run alone.  No host synchronisation. */
int kda_plan_varlen(const int32_t* cu_seqlens, int32_t N, int32_t T, int32_t chunk,
                    int32_t* chunk_indices, int32_t* chunk_offsets, kda_stream_t stream);

/* Debug check of device cu_seqlens (cu[0] == 0, non-decreasing, cu[N] == T).
 * SYNCHRONISES the stream and copies N+1 ints to the host.  Returns KDA_OK or
 * KDA_ERR_INVALID (KDA_ERR_HIP if the copy fails).
 * (torchtitan PR #4347, Performance and the Qwen3.5 paragraph: a device-to-host
 * read of the offsets in every layer was the cost that PR removed, so the
 * compute calls never read cu_seqlens on the host; their well-formedness is a
 * documented precondition, and this separate call checks it in tests.) */
int kda_check_cu_seqlens(const int32_t* cu_seqlens, int32_t N, int32_t T, kda_stream_t stream);

/* Workspace bytes needed by kda_fwd / kda_bwd for this descriptor (0 if the
 * descriptor is invalid; kda_last_error says why).  The caller allocates the
 * workspace once and passes it to every call; the library allocates nothing.
 * ("Pure KDA 300M on Primus" guide, Troubleshooting, "Out-of-memory at iter 1":
 * a kernel that allocates its own copies of q/k/v doubles their activation
 * memory; here every buffer, scratch included, is the caller's.)  For packed
 * rows pass B = 1 and N = the number of documents: the size then covers
 * kda_max_chunks(T, N, 64) chunks. */
size_t kda_fwd_workspace(const kda_desc* desc);
size_t kda_bwd_workspace(const kda_desc* desc);

/* Introspection of the workspace layout (host only; no device access): the
 * arrays that kda_fwd (backward = 0) or kda_bwd and a saving kda_fwd
 * (backward = 1) keep in the workspace for this descriptor, in workspace
 * order -- the name, byte offset and byte size of each.  Fills at most `cap`
 * entries of the arrays given (any of them may be null) and returns the number
 * of arrays, or -1 if the descriptor is invalid (kda_last_error says why).
 * The first 256 bytes of a workspace hold no array (offset 0 marks an absent
 * one inside the library).  For tests and tools that check the layout. */
int kda_debug_ws_layout(const kda_desc* desc, int backward, const char** names, size_t* offsets,
                        size_t* bytes, int cap);

/* Forward: o and the final states hT of the recurrence at the top of this
 * file, in chunked form (openkimi README, What is implemented: the chunk_kda
 * row, with fused Q/K norm, decay gate and beta; torchtitan PR #4347,
 * description: the recurrence takes cu_seqlens so that the state resets at
 * every document start).  Errors: KDA_ERR_INVALID / _UNSUPPORTED /
 * _WORKSPACE before any launch, outputs untouched; KDA_ERR_HIP if a launch
 * fails.
 *   q, k        [B,T,H,dk] dtype  (raw if KDA_F_QK_L2NORM)
 *   v           [B,T,H,dv] dtype
 *   g           [B,T,H,dk] fp32 log-decay (f if KDA_F_GATE_IN_KERNEL)
 *   beta        [B,T,H]    fp32 (logits if KDA_F_BETA_LOGITS)
 *   A_log       [H] fp32, dt_bias [H,dk] fp32: required iff KDA_F_GATE_IN_KERNEL
 *   h0          [N,H,dk,dv] fp32 initial states, nullable (= 0)
 *   cu_seqlens, chunk_indices, chunk_offsets: all null (dense) or all set
 *               (packed; B == 1; tables from kda_plan_varlen)
 *   o           [B,T,H,dv] out_dtype
 *   hT          [N,H,dk,dv] fp32 final states, nullable
 *   ws, ws_bytes  workspace of at least kda_fwd_workspace(desc) bytes */
int kda_fwd(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const float* A_log, const float* dt_bias, const float* h0,
            const int32_t* cu_seqlens, const int32_t* chunk_indices,
            const int32_t* chunk_offsets, void* o, float* hT, void* ws, size_t ws_bytes,
            kda_stream_t stream);

/* Forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, semantics and kernels as kda_fwd,
 * minus ws / ws_bytes: the workspace is a fixed scratch array of
 * KDA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, allocated
 * when the library's code is loaded on that GPU and held until the process
 * ends.  The call allocates and frees nothing.
 *   - kda_fwd_workspace(desc) must not exceed KDA_NOALLOC_SCRATCH_BYTES, else
 *     KDA_ERR_UNSUPPORTED (before any launch).  At dk = 32, dv = 64 that is
 *     about 1,200 chunk-heads, e.g. 8,192 tokens x 8 heads.
 *   - KDA_F_SAVE_FOR_BWD, KDA_F_FWD_SAVED and KDA_F_DH0_ONLY are refused
 *     (KDA_ERR_INVALID): the scratch does not outlive the call.
 *   - The stream's device must be the current device.  The first call on a
 *     device looks up that device's scratch address (hipGetSymbolAddress);
 *     make one call outside any graph capture first.
 *   - Every call on one GPU shares that GPU's scratch: calls that may overlap
 *     on one GPU (other streams, other threads) race and must be serialised
 *     by the caller.  No part of the scratch needs to start at zero: each call
 *     writes every scratch value before reading it.
 *   - With kda_timing_enable(1) the timing hooks create events; leave timing
 *     off where nothing may be allocated. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_fwd_noalloc(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, const float* A_log, const float* dt_bias, const float* h0,
                    const int32_t* cu_seqlens, const int32_t* chunk_indices,
                    const int32_t* chunk_offsets, void* o, float* hT, kda_stream_t stream);

/* Backward of kda_fwd with respect to every input it was given (openkimi
 * README, What is implemented: the chunk_kda row is forward and backward, with
 * the exact fp32-state recurrence as its reference; Profiling and H100
 * acceptance: gradients are compared with that reference, and decay-gradient
 * accuracy is the acceptance criterion).  Errors as kda_fwd.
 *   inputs as kda_fwd, plus
 *   d_o         [B,T,H,dv] dtype upstream gradient of o
 *   dhT         [N,H,dk,dv] fp32 upstream gradient of hT, nullable (= 0)
 *   dq, dk      [B,T,H,dk] out_dtype   (w.r.t. raw q, k if KDA_F_QK_L2NORM)
 *   dv          [B,T,H,dv] out_dtype
 *   dg          [B,T,H,dk] fp32        (w.r.t. f if KDA_F_GATE_IN_KERNEL)
 *   dbeta       [B,T,H]    fp32        (w.r.t. logits if KDA_F_BETA_LOGITS)
 *   dh0         [N,H,dk,dv] fp32, nullable
 *   dA_log [H], ddt_bias [H,dk] fp32: required iff KDA_F_GATE_IN_KERNEL;
 *               sums over all tokens, reduced in a fixed order (deterministic)
 *   ws, ws_bytes  workspace of at least kda_bwd_workspace(desc) bytes */
int kda_bwd(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const float* A_log, const float* dt_bias, const float* h0,
            const int32_t* cu_seqlens, const int32_t* chunk_indices,
            const int32_t* chunk_offsets, const void* d_o, const float* dhT, void* dq, void* dk,
            void* dv, float* dg, float* dbeta, float* dh0, float* dA_log, float* ddt_bias,
            void* ws, size_t ws_bytes, kda_stream_t stream);

/* One-token recurrent decode for B sequences (one iteration of the token
 * recurrence above; FlashKDA is the inference-only prior art named in the
 * openkimi README's FlashQLA paragraph).
 *   q, k   [B,H,dk] dtype (raw if KDA_F_QK_L2NORM); v [B,H,dv] dtype
 *   g      [B,H,dk] fp32 (f if KDA_F_GATE_IN_KERNEL); beta [B,H] fp32
 *   A_log, dt_bias as in kda_fwd
 *   h      [B,H,dk,dv] fp32 state, updated IN PLACE
 *   o      [B,H,dv] out_dtype, = scale * h_new^T q */
int kda_step(int32_t B, int32_t H, int32_t dk, int32_t dv, kda_dtype dtype, kda_dtype out_dtype,
             float scale, uint32_t flags, const void* q, const void* k, const void* v,
             const float* g, const float* beta, const float* A_log, const float* dt_bias,
             float* h, void* o, kda_stream_t stream);

/* ----------------------------------------------------------------------------
 * Context parallelism, every supported (dk, dv) (the one-GPU part of splitting a long
 * row over devices; the pages pack documents instead -- Packing PR -- and show
 * no context parallelism for KDA).  A chunk maps the state entering it
 * affinely to the state leaving it, so a segment of chunks does too:
 * h_out = M h_in + c, with c = kda_fwd's hT for h0 = 0.
 * kda_segment_maps: M [N,H,dk,dk] fp32 of every sequence (or packed document)
 *   of the call: the product of its chunks' transition matrices, first chunk
 *   rightmost (the identity for an empty one).  Inputs and flags as kda_fwd
 *   (no h0); ws of at least kda_fwd_workspace(desc) bytes.
 * kda_state_scan: chains R segments, H heads ((dk, dv) as kda_fwd supports):
 *   transpose = 0:  x = x0 (nullable = 0); for r = 0 .. R-1: x_in[r] = x; x = M_r x + c_r
 *   transpose = 1:  x = x0; for r = R-1 .. 0: x_in[r] = x; x = M_r^T x + c_r
 *   x_out (nullable) receives the final x.  M [R,H,dk,dk], c, x_in [R,H,dk,dv],
 *   x0, x_out [H,dk,dv], all fp32.  Forward: c_r = the segments' hT from h0 = 0,
 *   x0 = the row's h0; x_in[r] is then segment r's true h0 and x_out the row's hT.
 *   Backward: c_r = the segments' dh0 from kda_bwd with dhT = 0, x0 = the row's
 *   dhT; x_in[r] is then segment r's true dhT and x_out the row's dh0. */
int kda_segment_maps(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                     const int32_t* chunk_indices, const int32_t* chunk_offsets, float* M, void* ws,
                     size_t ws_bytes, kda_stream_t stream);
int kda_state_scan(int32_t R, int32_t H, int32_t dk, int32_t dv, int32_t transpose, const float* M,
                   const float* c, const float* x0, float* x_in, float* x_out, kda_stream_t stream);

/* ----------------------------------------------------------------------------
 * Short causal depthwise convolution, the step before KDA in its layer
 * ("Pure KDA 300M on Primus" guide, Overview: kernel size 4, depthwise, on
 * the concatenated q/k/v channels; Troubleshooting: [B, T, D] is the native
 * layout; torchtitan PR #4347, description: with document offsets the window
 * resets at every document start).  Readings: an optional bias and an
 * optional SiLU, which the pages do not fix.
 *   z[b,t,c] = sum_{i<W} w[c,i] x[b, t-(W-1)+i, c]  over positions of the same
 *              document (earlier positions count as zero) + bias[c]
 *   y        = z, or SiLU(z) with KDA_CONV_SILU
 *   x, y       [B,T,D] dtype / out_dtype, D a multiple of 8
 *   w          [D,W] fp32, W in 1..4; bias [D] fp32, nullable (= 0)
 *   cu_seqlens [N+1] int32 document offsets, nullable (dense rows); needs B == 1
 * Backward: dx [B,T,D] out_dtype; dw [D,W] and dbias [D] (nullable) fp32, sums
 * over all tokens in a fixed order (deterministic); ws of at least
 * kda_conv_bwd_workspace(B,T,D,W) bytes (0 = invalid sizes). */
enum { KDA_CONV_SILU = 1u << 0 };
int kda_conv_fwd(int32_t B, int32_t T, int32_t D, int32_t W, kda_dtype dtype, kda_dtype out_dtype,
                 uint32_t flags, const void* x, const float* w, const float* bias,
                 const int32_t* cu_seqlens, int32_t N, void* y, kda_stream_t stream);
size_t kda_conv_bwd_workspace(int32_t B, int32_t T, int32_t D, int32_t W);
int kda_conv_bwd(int32_t B, int32_t T, int32_t D, int32_t W, kda_dtype dtype, kda_dtype out_dtype,
                 uint32_t flags, const void* x, const float* w, const float* bias,
                 const int32_t* cu_seqlens, int32_t N, const void* dy, void* dx, float* dw,
                 float* dbias, void* ws, size_t ws_bytes, kda_stream_t stream);

/* ----------------------------------------------------------------------------
 * Gated RMS norm of the KDA output, the step after KDA in its layer (openkimi
 * README, Profiling and H100 acceptance: the KDA output goes through a fused
 * RMSNorm and a sigmoid gate; Primus guide, Overview: per-head output gate,
 * RMSNorm eps 1e-6).  Per row of dv values (one token and head):
 *   y = o (mean(o^2) + eps)^{-1/2} * weight * sigmoid(gate)
 *   o, gate, y   [rows, dv] dtype / out_dtype (rows = B*T*H), dv in {32, 64, 128}
 *   weight       [dv] fp32, shared by the heads (reading: one g_norm of head_v_dim)
 * Backward: d_o, dgate [rows, dv] out_dtype; dweight [dv] fp32, a sum over all
 * rows in a fixed order; ws of at least kda_gnorm_bwd_workspace(rows, dv) bytes. */
int kda_gnorm_fwd(int64_t rows, int32_t dv, kda_dtype dtype, kda_dtype out_dtype, float eps,
                  const void* o, const void* gate, const float* weight, void* y, kda_stream_t stream);
size_t kda_gnorm_bwd_workspace(int64_t rows, int32_t dv);
int kda_gnorm_bwd(int64_t rows, int32_t dv, kda_dtype dtype, kda_dtype out_dtype, float eps,
                  const void* o, const void* gate, const float* weight, const void* dy, void* d_o,
                  void* dgate, float* dweight, void* ws, size_t ws_bytes, kda_stream_t stream);

/* Opt-in per-kernel timing for benchmarks.  kda_timing_enable(1) clears the
 * record and brackets every later kernel launch of this library with a pair
 * of hipEvents on the launch stream (enable(0) stops; pending events are
 * dropped).  kda_timing_collect() waits for the recorded events (it
 * SYNCHRONISES on them) and adds their durations to per-kernel totals, read
 * with kda_timing_count() / kda_timing_get(i, &name, &launches, &total_ms);
 * `name` stays valid until the next enable call.  Kernel names: plan, step,
 * fwd_intra, fwd_scan, bwd_dh, bwd_chunk, bwd_dv, bwd_dk, bwd_gate_sum,
 * conv_fwd, conv_bwd, conv_wsum, gnorm_fwd, gnorm_bwd, gnorm_wsum, seg_map, state_scan. */
int kda_timing_enable(int on);
int kda_timing_collect(void);
int kda_timing_count(void);
int kda_timing_get(int i, const char** name, int64_t* launches, double* total_ms);

/* Static text for a status code, and the thread-local message of the last
 * failing call on this thread ("" if none). */
const char* kda_status_str(int status);
const char* kda_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
