// Host-side interface between the C ABI layer (kda_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
  const void *q, *k, *v, *g, *beta;
  float* state;
  void* o;
  int units;  // B * H
  int dk, dv;
  bool f32;
  void* stream;
};

struct PrefillArgs {
  const void *q, *k, *v, *g, *beta;
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
};

// intra-chunk kernel launch (kda_intra.hip)
struct IntraLaunch {
  const void *q, *k, *v, *g, *beta;
  const int32_t* cu;
  const int32_t* chunk0;
  unsigned char* records;
  int num_seqs, H, T, nch;
  int dk, dv, chunk;
  bool f32;
  int grid;
  void* stream;
};

// chain kernel launch (kda_chain.hip)
struct ChainLaunch {
  const unsigned char* records;
  const float* h0;
  void* o;
  float* hT;
  const int32_t* cu;
  const int32_t* chunk0;
  int units, H, T, nch;
  int dk, dv, chunk, ws;
  bool f32;
  void* stream;
};

hipError_t launch_decode_step(const DecodeArgs& a);
hipError_t launch_intra(const IntraLaunch& L);
hipError_t launch_chain(const ChainLaunch& L);
hipError_t launch_chunk_map(const int32_t* cu, int num_seqs, int T, int C, int32_t* chunk0, void* stream);

// Prefill: supported shape?  workspace bytes?  launch (hipErrorInvalidValue: unsupported shape).
bool chunked_forward_supported(bool f32, int dk, int dv, int chunk);
size_t chunked_forward_workspace(bool f32, int dk, int dv, int chunk, int64_t max_chunks, int H, int num_seqs,
                                 bool varlen);
hipError_t launch_chunked_forward(const PrefillArgs& a);

}  // namespace kda
