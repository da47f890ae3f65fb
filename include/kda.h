/*
 * kda.h -- C ABI of libkda.so, Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).
 *
 * KDA is the gated delta-rule linear attention of Kimi K3 (technical-report
 * page, "Quick answer", "Architecture at a glance" and FAQ "What is Kimi Delta
 * Attention?"; architecture blog, "Kimi Delta Attention: the linear core").
 * Per (sequence, head) it carries a fixed-size state S (d_k x d_v, fp32) and,
 * for every token t,
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,     o_t = S_t^T q_t
 *
 * with g_t the per-key-channel log-decay (the channel-wise forget gate; the
 * pages bound it below through a scaled sigmoid, so the library expects
 * -5 <= g <= 0 and takes g as given), beta_t a per-(token, head) write
 * strength in [0, 1], and no query scaling.  o_t is read after the update.
 * The prefill entry points evaluate this in its chunkwise form (the pages'
 * "chunkwise algorithm" on specialised diagonal-plus-low-rank transitions);
 * the result equals the token-by-token recurrence up to rounding and does not
 * depend on the chunk size beyond rounding.
 *
 * Conventions common to every entry point
 *  - Every pointer is device memory owned by the caller.  The library never
 *    allocates or frees device memory and keeps no state between calls.
 *  - All work is enqueued on `hip_stream` (a hipStream_t; NULL = the null
 *    stream).  No call synchronises the host, copies between host and device,
 *    or allocates.  Results are visible once the caller synchronises.
 *  - Arguments are validated before anything is enqueued: an invalid call
 *    returns a nonzero status and has no side effects.  A failed launch
 *    returns KDA_ERR_HIP.  Faults during execution surface at the caller's
 *    synchronisation.
 *  - Layouts are row-major and contiguous:
 *      q, k, g   [B, T, H, d_k]      v, o   [B, T, H, d_v]      beta [B, T, H]
 *      h0, hT, state   [B, H, d_k, d_v] fp32
 *    q, k, v, g, beta and o share one dtype (kda_dtype); states are fp32.
 *  - Supported: d_k, d_v in {64, 128}; chunk in {16, 32, 64}; fp32 or bf16;
 *    any T >= 0; pointers 16-byte aligned.  Anything else returns
 *    KDA_ERR_UNSUPPORTED.
 *  - Deterministic: no atomics; repeated calls give bitwise-identical results.
 *  - Thread-safe: calls share no mutable state.
 *  - Inputs are expected in the documented envelope (-5 <= g <= 0,
 *    0 <= beta <= 1, |q|, |k| of order 1).  Outside it the result is
 *    unspecified; NaN or Inf in an input propagates to o and hT.
 *
 * Debug build (libkda_debug.so: the same sources, kda_api.hip compiled with
 * KDA_DEBUG_CHECKS; kda_debug_checks() returns 1)
 *  - Every entry point that takes g and beta first checks them against the
 *    envelope on the GPU: each element of g in [-5, 0] (skipped where the
 *    fused gate forms g from a pre-activation, which keeps it there by
 *    construction) and each element of beta in [0, 1]; NaN and Inf fail.  A
 *    violation returns KDA_ERR_ENVELOPE and nothing else is enqueued.
 *  - To read the check's result the debug build synchronises `hip_stream`
 *    once per call (unlike the release build, which never synchronises), so it
 *    is for diagnosis, not for graph capture or timing.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of q, k, v, g, beta and o (states are always fp32) */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null pointer, negative size, misaligned pointer, bad cu_seqlens bound */
  KDA_ERR_UNSUPPORTED = 2, /* valid but outside the supported shapes */
  KDA_ERR_WORKSPACE = 3,   /* workspace smaller than the size query returned */
  KDA_ERR_HIP = 4,         /* a HIP launch or runtime call failed */
  KDA_ERR_ENVELOPE = 5     /* debug build only: g or beta outside the documented envelope */
} kda_status;

/* Static description of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int kda_version(void);

/* 1 in the debug build (the envelope checks above), 0 in the release build. */
int kda_debug_checks(void);

/*
 * Bytes of device workspace kda_chunked_forward needs for this shape
 * (0 = none; the workspace arguments may then be NULL / 0).
 */
size_t kda_chunked_forward_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt);

/*
 * How kda_chunked_forward lays out its state chain on the current device for
 * this shape: *value_slice = value columns of the state per workgroup (16 or
 * 32); *segments = the number of segments every sequence is split into (1 =
 * none: the chain runs over whole sequences); *segment_chunks = chunks per
 * segment (0 when *segments is 1); *summary_slice = state columns per
 * workgroup of the segment summary pass (0 when *segments is 1).  Sequences
 * are split only when (sequence, head, value slice) alone would leave compute
 * units idle; the split costs a summary pass and a combine but runs the chain
 * on more workgroups.  Any output pointer may be NULL.  The workspace size
 * query accounts for the plan, so query, plan and call must use the same
 * device.
 */
kda_status kda_chunked_forward_plan(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt,
                                    int* value_slice, int* segments, int* segment_chunks, int* summary_slice);

/*
 * Optional steps fused on either side of the recurrence, for the *_fused entry
 * points (a NULL kda_fusion pointer, or all fields zero, means none):
 *  - gate_x: the gate pre-activation, laid out and typed like g.  The kernel
 *    then forms the log-decay through a scaled sigmoid, g = -gate_scale *
 *    sigmoid(gate_x) (technical-report page, "Architecture at a glance": the
 *    lower bound on the log-decay), and the g argument is not read (may be
 *    NULL).  gate_scale must lie in (0, 5]: the kernels rely on g >= -5.
 *  - normalize_qk: nonzero L2-normalises q and k over d_k per (token, head),
 *    x / sqrt(sum x^2 + 1e-12), in fp32 in the kernel.
 *  - out_gate: an output gate z laid out and typed like o; o is multiplied by
 *    z elementwise before it is stored (same page: the input-dependent output
 *    gate; z is taken as given -- its projection needs trained weights).
 * All pointers are device memory, 16-byte aligned.
 */
typedef struct {
  const void* gate_x;
  float gate_scale;
  int normalize_qk;
  const void* out_gate;
} kda_fusion;

/*
 * Chunked prefill over B sequences of T tokens each.
 *   q, k, g [B,T,H,d_k], v [B,T,H,d_v], beta [B,T,H]   (dtype dt)   in
 *   h0 [B,H,d_k,d_v] fp32                               in, or NULL for a zero initial state
 *   o  [B,T,H,d_v]   (dtype dt)                          out
 *   hT [B,H,d_k,d_v] fp32                               out, or NULL if not wanted
 * hT may be the same pointer as h0 (the state is read before it is
 * overwritten); any other overlap between outputs and inputs is undefined.
 * T = 0 writes hT = h0 (or zeros) and nothing else.
 * chunk: tokens per chunk of the chunkwise form (a performance knob).
 */
kda_status kda_chunked_forward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v, int chunk,
                               kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * kda_chunked_forward for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, layouts, results and errors as
 * kda_chunked_forward, without the workspace: the scratch it needs (the
 * per-chunk records and segment states; kda_chunked_forward_workspace_bytes
 * gives its size) lives in a fixed device buffer of KDA_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held from the first use of the library on
 * that GPU until the process ends.  The call allocates nothing.
 *   KDA_ERR_WORKSPACE: the shape needs more than KDA_NOALLOC_SCRATCH_BYTES of
 *   scratch (use kda_chunked_forward with a workspace, or split the call).
 *   KDA_ERR_HIP also if the runtime cannot give the buffer's device address.
 * Every call on one GPU uses that GPU's single buffer: calls on one stream are
 * ordered, but calls whose executions overlap on one GPU (different streams,
 * host threads) race on it and give unspecified results.  The kernels write
 * every scratch byte they read before reading it, so the contents a previous
 * call left behind are never used and nothing is cleared.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_chunked_forward_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                       const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                       int chunk, kda_dtype dt, void* hip_stream);

/*
 * kda_chunked_forward that also keeps the recurrent state at fixed token
 * intervals: the prefix states a serving cache stores so that a repeated
 * prompt resumes from the state instead of being prefilled again (a recurrent
 * state has no per-token KV slabs to replay: how-K3-works page, "KDA: a fixed
 * memory instead of a growing bill"; architecture-explained page, "Kimi Delta
 * Attention: Scaling Attention Beyond the Trillion-Parameter Regime").
 *   states [B,H,T/state_every,d_k,d_v] fp32 out (16-byte aligned): entry j is the
 *          state after the first (j+1)*state_every tokens of the sequence, i.e.
 *          hT of a call on that prefix; passing it as h0 resumes from there.
 *   state_every: a positive multiple of chunk.
 * states may be NULL (then state_every is ignored and this is
 * kda_chunked_forward).  Any overlap of states with another argument is
 * undefined.  Other arguments, the workspace and errors as kda_chunked_forward.
 */
kda_status kda_chunked_forward_with_states(const void* q, const void* k, const void* v, const void* g,
                                           const void* beta, const float* h0, void* o, float* hT, float* states,
                                           int state_every, int B, int T, int H, int d_k, int d_v, int chunk,
                                           kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * kda_chunked_forward with the fused steps of *fusion (see kda_fusion); the
 * arguments, workspace and errors are otherwise those of kda_chunked_forward.
 * KDA_ERR_INVALID_ARG also for a gate_scale outside (0, 5] with gate_x, or a
 * misaligned gate_x / out_gate.
 */
kda_status kda_chunked_forward_fused(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                     const float* h0, void* o, float* hT, const kda_fusion* fusion, int B, int T,
                                     int H, int d_k, int d_v, int chunk, kda_dtype dt, void* workspace,
                                     size_t workspace_bytes, void* hip_stream);

/*
 * kda_chunked_forward with q, k and v in the OCP Microscaling FP8 format
 * (MXFP8): the pages train K3 with MXFP8 activations (how-K3-works page, "The
 * systems layer": quantisation-aware training with MXFP4 weights and MXFP8
 * activations), so the inputs of the recurrence may arrive in it.
 *   q, k     [B,T,H,d_k] uint8: FP8 E4M3 codes (sign, 4 exponent bits with
 *            bias 7, 3 mantissa bits; no infinities; 0x7F / 0xFF are NaN)
 *   v        [B,T,H,d_v] uint8: FP8 E4M3 codes
 *   q_scale, k_scale [B,T,H,d_k/32], v_scale [B,T,H,d_v/32] uint8: E8M0
 *            scale codes, one per block of 32 consecutive channels of a
 *            (token, head); code s stands for 2^(s-127), 255 is NaN
 * Element x of a block with scale code s stands for E4M3(x) * 2^(s-127).
 * g, beta and o are bf16, h0 / hT fp32, all as for kda_chunked_forward with
 * KDA_BF16.  The kernels decode q, k and v as they load them; every decoded
 * value of magnitude >= 2^-133 is a bf16 value, so the call computes what
 * kda_chunked_forward (KDA_BF16) computes on the decoded q, k, v.  Workspace:
 * kda_chunked_forward_workspace_bytes(..., KDA_BF16).  q, k, v 16-byte
 * aligned; scales have no alignment requirement.  Same shapes, errors and
 * stream semantics as kda_chunked_forward (KDA_ERR_INVALID_ARG also for a NULL
 * scale pointer when B * T > 0).
 */
kda_status kda_chunked_forward_mxfp8(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                     const void* v, const void* v_scale, const void* g, const void* beta,
                                     const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                     int chunk, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * kda_chunked_forward with both state snapshots (states, state_every: see
 * kda_chunked_forward_with_states; states may be NULL) and fused steps
 * (fusion: see kda_fusion; may be NULL).
 */
kda_status kda_chunked_forward_ex(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                  const float* h0, void* o, float* hT, float* states, int state_every,
                                  const kda_fusion* fusion, int B, int T, int H, int d_k, int d_v, int chunk,
                                  kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Profiling form of kda_chunked_forward: the same arguments, checks and
 * results, plus kernel_ms[2] (host memory, non-NULL), which receives the
 * durations in milliseconds of the two stages of the call -- [0] the
 * intra-chunk kernel (gate cumulative sums, the UT/WY transform and the
 * chunk-local products; architecture blog, "Kimi Delta Attention: the linear
 * core"), [1] the state chain (the sequential recurrence: one chain kernel, or
 * for a segmented plan the summary pass, the combine and the chain) -- measured
 * with HIP events recorded on hip_stream around each.  It creates and destroys
 * its events and synchronises with the stream before returning, so it is for
 * measurement, not for a launch loop.  kernel_ms is zeroed when nothing runs.
 */
kda_status kda_chunked_forward_profiled(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                        const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                        int chunk, kda_dtype dt, void* workspace, size_t workspace_bytes,
                                        void* hip_stream, float* kernel_ms);

/*
 * Packed variable-length prefill: num_seqs sequences concatenated along the
 * token axis (tensors as above with B = 1 and T = T_total); sequence n covers
 * tokens [cu_seqlens[n], cu_seqlens[n+1]).  cu_seqlens is an int32 device
 * array of num_seqs + 1 non-decreasing offsets with cu_seqlens[0] = 0 and
 * cu_seqlens[num_seqs] = T_total; it is read on the device only (no host
 * synchronisation).  max_seqlen must bound every sequence length; it sizes
 * nothing on the host and may be an over-estimate.  Chunks restart at every
 * sequence start and no state crosses a sequence boundary.
 *   h0, hT [num_seqs, H, d_k, d_v] fp32 (either may be NULL; hT may equal h0).
 * Offsets that violate the contract above give unspecified results for the
 * affected sequences but never access memory outside [0, T_total).
 */
kda_status kda_chunked_forward_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                      const float* h0, void* o, float* hT, const int32_t* cu_seqlens, int num_seqs,
                                      int T_total, int max_seqlen, int H, int d_k, int d_v, int chunk, kda_dtype dt,
                                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * kda_chunked_forward_varlen with state snapshots (see
 * kda_chunked_forward_with_states): states [num_seqs,H,max_seqlen/state_every,
 * d_k,d_v] fp32; entry j of sequence n is its state after (j+1)*state_every
 * tokens; entries past a sequence's length are left untouched.
 */
kda_status kda_chunked_forward_varlen_with_states(const void* q, const void* k, const void* v, const void* g,
                                                  const void* beta, const float* h0, void* o, float* hT,
                                                  float* states, int state_every, const int32_t* cu_seqlens,
                                                  int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v,
                                                  int chunk, kda_dtype dt, void* workspace, size_t workspace_bytes,
                                                  void* hip_stream);

/*
 * kda_chunked_forward_varlen with both state snapshots (see
 * kda_chunked_forward_varlen_with_states; states may be NULL) and fused steps
 * (see kda_fusion; gate_x laid out like g and out_gate like o; may be NULL).
 */
kda_status kda_chunked_forward_varlen_ex(const void* q, const void* k, const void* v, const void* g,
                                         const void* beta, const float* h0, void* o, float* hT, float* states,
                                         int state_every, const kda_fusion* fusion, const int32_t* cu_seqlens,
                                         int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v, int chunk,
                                         kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes kda_chunked_forward_varlen needs (0 = none). */
size_t kda_chunked_forward_varlen_workspace_bytes(int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v,
                                                  int chunk, kda_dtype dt);

/*
 * One decode step for B sequences (one token each), updating the fp32 state
 * in place (the fixed-size state that replaces a growing KV cache: architecture
 * blog, "Why the attention stack is the story"; how-K3-works page, "KDA: a
 * fixed memory instead of a growing bill").
 *   q, k, g [B,H,d_k], v [B,H,d_v], beta [B,H]   (dtype dt)   in
 *   state [B,H,d_k,d_v] fp32                      in/out
 *   o [B,H,d_v] (dtype dt)                        out
 * The state is read and written once; o needs no second pass over it.
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta, float* state,
                           void* o, int B, int H, int d_k, int d_v, kda_dtype dt, void* hip_stream);

/*
 * kda_decode_step with the fused steps of *fusion (see kda_fusion): gate_x
 * [B,H,d_k], out_gate [B,H,d_v].  Otherwise as kda_decode_step.
 */
kda_status kda_decode_step_fused(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                 float* state, void* o, const kda_fusion* fusion, int B, int H, int d_k, int d_v,
                                 kda_dtype dt, void* hip_stream);

/*
 * Backward of kda_chunked_forward, for training with KDA (technical-report
 * page, "Training"; the pages give no backward, so it is the chain rule through
 * the chunkwise form the forward computes).  Given the adjoints d_o = dL/do
 * and dhT = dL/dhT of a loss L, it returns
 *   dq, dk, dg [B,T,H,d_k], dv [B,T,H,d_v], dbeta [B,T,H]   (dtype dt)   out
 *   dh0 [B,H,d_k,d_v] fp32 (NULL: not written)                          out
 * from the forward's inputs q, k, v, g, beta, h0 (as in kda_chunked_forward;
 * h0 NULL = zero start) and
 *   d_o [B,T,H,d_v] (dtype dt), dhT [B,H,d_k,d_v] fp32 (NULL = zero)    in
 * The forward is recomputed inside the call (nothing is kept from an earlier
 * forward call).  Supported: bf16 or fp32 with d_k, d_v in {64, 128}; chunk
 * in {16, 32, 64}; anything else returns KDA_ERR_UNSUPPORTED.  workspace: kda_chunked_backward_workspace_bytes(...)
 * bytes, 256-byte aligned, caller-owned (it holds the recomputed per-chunk
 * records and states and the adjoint states).  Every output is written, none
 * is read; outputs must not overlap inputs.  Invalid calls return an error
 * before anything is launched.
 */
kda_status kda_chunked_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                const float* h0, const void* d_o, const float* dhT, void* dq, void* dk, void* dv,
                                void* dg, void* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v, int chunk,
                                kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes kda_chunked_backward needs (0 = unsupported shape). */
size_t kda_chunked_backward_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt);

/*
 * Backward of kda_chunked_forward_varlen: the packed sequences of
 * kda_chunked_forward_varlen (tensors as in kda_chunked_backward with B = 1
 * and T = T_total; cu_seqlens, num_seqs, T_total and max_seqlen as in
 * kda_chunked_forward_varlen), with h0, dhT and dh0 per sequence
 * [num_seqs,H,d_k,d_v] fp32.  Every sequence's gradients are those of its own
 * <d_o, o> + <dhT, hT>; no adjoint crosses a sequence boundary, and an empty
 * sequence gets dh0 = dhT.  Same domain, errors, ownership and stream
 * semantics as kda_chunked_backward.  workspace:
 * kda_chunked_backward_varlen_workspace_bytes(...) bytes, 256-byte aligned.
 */
kda_status kda_chunked_backward_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                       const float* h0, const void* d_o, const float* dhT, void* dq, void* dk,
                                       void* dv, void* dg, void* dbeta, float* dh0, const int32_t* cu_seqlens,
                                       int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v, int chunk,
                                       kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes kda_chunked_backward_varlen needs (0 = unsupported shape). */
size_t kda_chunked_backward_varlen_workspace_bytes(int num_seqs, int T_total, int max_seqlen, int H, int d_k,
                                                   int d_v, int chunk, kda_dtype dt);

/*
 * A training step without the recompute: the forward keeps what the backward
 * needs, the backward uses it.  kda_chunked_forward_train computes o and hT
 * exactly as kda_chunked_forward (the same kernels; bitwise the same results)
 * and also leaves, in the caller-owned `saved` buffer, every (chunk, head)
 * record of the chunkwise form and the state at every chunk start (in the
 * dtype dt).  kda_chunked_backward_saved then returns the gradients
 * kda_chunked_backward returns for the same inputs (bitwise the same) without
 * running the forward again.  The caller keeps `saved` unchanged, and passes
 * the same q, k, v, g, beta, h0 and shapes, between the two calls; the
 * library cannot check that.  Equal-length sequences; same domain, errors,
 * ownership and stream semantics as kda_chunked_backward.
 *   saved: kda_chunked_forward_train_saved_bytes(...) bytes, 256-byte aligned
 *   workspace (backward): kda_chunked_backward_saved_workspace_bytes(...)
 *     bytes, 256-byte aligned (the adjoint states and the state products)
 * The two together hold what kda_chunked_backward's own workspace holds, less
 * its recomputed o.
 */
kda_status kda_chunked_forward_train(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                     const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                     int chunk, kda_dtype dt, void* saved, size_t saved_bytes, void* hip_stream);

/* Bytes of the `saved` buffer kda_chunked_forward_train fills (0 = unsupported shape). */
size_t kda_chunked_forward_train_saved_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt);

kda_status kda_chunked_backward_saved(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                      const float* h0, const void* d_o, const float* dhT, void* dq, void* dk,
                                      void* dv, void* dg, void* dbeta, float* dh0, int B, int T, int H, int d_k,
                                      int d_v, int chunk, kda_dtype dt, const void* saved, size_t saved_bytes,
                                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes kda_chunked_backward_saved needs (0 = unsupported shape). */
size_t kda_chunked_backward_saved_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
