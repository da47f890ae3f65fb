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
  void* stream;
};

hipError_t launch_decode_step(const DecodeArgs& a);

// Returns hipErrorInvalidValue when no kernel instance covers the shape.
hipError_t launch_chunked_forward(const PrefillArgs& a);
bool chunked_forward_supported(bool f32, int dk, int dv, int chunk);

}  // namespace kda
