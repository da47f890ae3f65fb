// Host-side interface between the C ABI layer (kda_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Optional steps fused on either side of the recurrence (all off by default):
//   gate_scale > 0: the g pointer holds the gate pre-activation x, and g = -gate_scale sigmoid(x);
//   normalize_qk:   q and k are L2-normalised over d_k per (token, head) in the kernel;
//   out_gate:       o is multiplied elementwise by this tensor (laid out and typed like o).
struct Fusion {
  float gate_scale = 0.f;
  bool normalize_qk = false;
  const void* out_gate = nullptr;
};

struct DecodeArgs {
  const void *q, *k, *v, *g, *beta;
  float* state;
  void* o;
  int units;  // B * H
  int dk, dv;
  bool f32;
  void* stream;
  Fusion fusion;
};

struct PrefillArgs {
  const void *q, *k, *v, *g, *beta;
  const uint8_t *q_scale = nullptr, *k_scale = nullptr, *v_scale = nullptr;  // non-NULL: q, k, v are MXFP8
  const float* h0;
  void* o;
  float* hT;
  const int32_t* cu_seqlens;  // device offsets [num_seqs + 1], or NULL for B equal-length sequences
  int num_seqs;               // B (cu_seqlens == NULL) or the number of packed sequences
  int T;                      // tokens per sequence (cu_seqlens == NULL) or T_total
  int H, dk, dv, chunk;
  bool f32;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  hipEvent_t* events = nullptr;  // optional: [3] recorded before the intra kernel, between the kernels, after the chain
  float* states = nullptr;       // optional state snapshots [num_seqs][H][max_states][dk][dv]
  int state_every = 0, max_states = 0;
  bool states_bf16 = false;      // with states_by_chunk: the states stored as bf16 (the bf16 backward)
  bool states_by_chunk = false;  // instead: state_every = chunk, the state after every full chunk at
                                 // its record's slot [(chunk) H + head][dk][dv] (the backward's layout)
  Fusion fusion;
};

// intra-chunk kernel launch (kda_intra.hip)
struct IntraLaunch {
  const void *q, *k, *v, *g, *beta;
  const uint8_t *qs = nullptr, *ks = nullptr, *vs = nullptr;  // non-NULL: q, k, v are MXFP8 (E4M3 codes)
  const int32_t* cu;
  const int32_t* chunk0;
  unsigned char* records;
  int num_seqs, H, T, nch;
  int dk, dv, chunk;
  bool f32;
  int grid;
  void* stream;
  float gate_scale = 0.f;  // > 0: g holds the gate pre-activation (Fusion)
  bool normalize_qk = false;
};

// chain kernel launch (kda_chain.hip)
struct ChainLaunch {
  const unsigned char* records;
  const float* h0;
  void* o;
  float* hT;
  const int32_t* cu;
  const int32_t* chunk0;
  const int32_t* order = nullptr;  // packed sequences longest first, or NULL
  int units, H, T, nch;
  int dk, dv, chunk, ws;
  bool f32;
  // segments (equal-length sequences only): nseg > 1 splits every (sequence, head) into segments of
  // seg_len chunks.  summary: run segments 0..nseg-2 from the zero state on the value columns and
  // from the identity on d_k extra columns, writing [b_g | M_g] to send; otherwise segment g starts
  // from sstart[unit][g] (all segments, the first included) and writes o, and the last writes hT.
  int nseg = 1, seg_len = 0;
  bool summary = false;
  bool wide = false;  // the wide kernel (bf16, chunk 64: 32-column chain waves, ws up to 128)
  const float* sstart = nullptr;  // [units][nseg][dk][dv]
  float* send = nullptr;          // [units][nseg - 1][dk][dv + dk]
  // optional state snapshots after every `every` tokens of each sequence (every: a multiple of
  // chunk): [units][max_states][dk][dv]
  float* states = nullptr;
  int every = 0, max_states = 0;
  bool states_by_chunk = false;  // every = chunk, the state after each full chunk at [(chunk) H + head]
  bool states_bf16 = false;      // the states stored as bf16 (the bf16 backward's chunk-start states)
  const void* out_gate = nullptr;  // o is multiplied by it elementwise (Fusion)
  void* stream;
};

// How the chain is laid out over the GPU: value-slice width, the segment split of long sequences
// whose (sequence, head, slice) count alone would leave compute units idle, and the column-slice
// width of the segment summaries (0 when the plan has no segments).
struct ChainPlan {
  int ws, nseg, seg_len, sum_ws;
  bool wide;  // chain_wide_kernel (bf16 records of 64-token chunks), else chain_kernel
};
ChainPlan chain_plan(bool f32, int64_t units, int nch, int dk, int dv, int chunk, bool varlen);

// Compute units of the current device (256 when none can be queried), cached per device.
int compute_units();

// Segment start states: sstart[u][0] = h0 (or 0), sstart[u][g + 1] = M_g sstart[u][g] + b_g
// (kda_chain.hip)
hipError_t launch_segment_combine(const float* h0, const float* send, float* sstart, int units, int nseg, int dk,
                                  int dv, void* stream);

hipError_t launch_decode_step(const DecodeArgs& a);
hipError_t launch_intra(const IntraLaunch& L);
hipError_t launch_chain(const ChainLaunch& L);
hipError_t launch_chunk_map(const int32_t* cu, int num_seqs, int T, int C, int32_t* chunk0, int32_t* order,
                            void* stream);

// Backward of the chunked prefill (kda_backward.hip): gradients of <dO, o> + <dhT, hT>.
struct BackwardArgs {
  const void *q, *k, *v, *g, *beta;
  const int32_t* cu_seqlens = nullptr;  // packed sequences (B = num_seqs, T = T_total), or NULL
  const float* h0;   // or NULL (zero)
  const void* dO;    // like o
  const float* dhT;  // or NULL (zero)
  void *dq, *dk_out, *dv_out, *dg, *dbeta;  // like q, k, v, g, beta
  float* dh0;        // or NULL (not written)
  int B, T, H, dk, dv, chunk;
  bool f32;
  void* workspace;
  void* stream;
  // training: what a forward-train call left (records, chunk map, chunk-start states), or NULL to
  // recompute the forward into the workspace
  const void* saved = nullptr;
};
bool chunked_backward_supported(bool f32, int dk, int dv, int chunk);
// the whole workspace of a backward that recomputes the forward
size_t chunked_backward_workspace(bool f32, int dk, int dv, int chunk, int num_seqs, int T, int H, bool varlen);
// the part of it a forward-train call fills (records, chunk map, chunk-start states), and the rest
// a backward from that saved part needs as its workspace
size_t chunked_backward_saved_bytes(bool f32, int dk, int dv, int chunk, int num_seqs, int T, int H, bool varlen);
size_t chunked_backward_own_bytes(bool f32, int dk, int dv, int chunk, int num_seqs, int T, int H, bool varlen);
hipError_t launch_chunked_backward(const BackwardArgs& a);
// the forward of a training step: o and hT as kda_chunked_forward, and the backward's saved part in
// `saved` (a.workspace is ignored; a.dO, the gradient pointers and a.dhT are not used)
hipError_t launch_forward_train(const BackwardArgs& a, void* saved, void* o, float* hT);

// Prefill: supported shape?  workspace bytes?  launch (hipErrorInvalidValue: unsupported shape).
bool chunked_forward_supported(bool f32, int dk, int dv, int chunk);
size_t chunked_forward_workspace(bool f32, int dk, int dv, int chunk, int64_t max_chunks, int H, int num_seqs,
                                 bool varlen);
hipError_t launch_chunked_forward(const PrefillArgs& a);
// the chunk map of a packed call inside its workspace (built by launch_chunked_forward)
void chunk_map_of(void* workspace, bool f32, int dk, int dv, int chunk, int64_t max_chunks, int H, int num_seqs,
                  int32_t** chunk0, int32_t** order);

}  // namespace kda
