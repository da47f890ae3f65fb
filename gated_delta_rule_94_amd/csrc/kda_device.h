// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4).
//
// Element types: inputs and outputs are fp32 or bf16 (stored as raw 16-bit
// patterns); all arithmetic is fp32.  fp32 -> bf16 uses the hardware
// round-to-nearest-even conversion.
//
// MFMA fragment conventions (wave64, 16x16 output tiles).  Lane l has
// lo = l % 16 and grp = l / 16.  The f32 accumulator of a 16x16 tile holds,
// in lane l, element D[4*grp + r][lo] for r = 0..3.  A-operand lanes hold row
// lo of A, B-operand lanes hold column lo of B, and lane group grp holds a
// slice of the contraction index.  Which contraction index a (grp, slot)
// carries is a choice of this library, made identically for A and B, so the
// product is independent of it.  The choice used everywhere is the
// "accumulator order": slot j of group grp in k-step s carries
//   bf16 16x16x32 : k = 32 s + 16 (j / 4) + 4 grp + (j % 4)     (j = 0..7)
//   fp32 16x16x4  : k = 16 (s / 4) + 4 grp + (s % 4)           (one slot)
//   bf16 16x16x16 : k = 4 grp + j                               (j = 0..3)
// With it an accumulator tile (or a pair of them) is directly a B operand
// contracting over the accumulator's rows, so chained products (the delta
// rule's U -> S update, S -> the next chunk) never leave registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Load / store one element of an fp32 or bf16 tensor as fp32.
template <bool F32>
__device__ __forceinline__ float ldg(const void* p, int64_t i) {
  if constexpr (F32) return static_cast<const float*>(p)[i];
  else return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <bool F32>
__device__ __forceinline__ void stg(void* p, int64_t i, float x) {
  if constexpr (F32) static_cast<float*>(p)[i] = x;
  else static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------------------------
// Operand policy: element type of staged operands and the MFMA used for dense contractions.
template <bool F32>
struct Op;

// bf16 operands, v_mfma_f32_16x16x32_bf16 (fp32 accumulate)
template <>
struct Op<false> {
  using E = __bf16;
  using Frag = bf16x8;
  static constexpr int KS = 32;  // contraction length of one MFMA
  // contraction index carried by slot j of lane group grp in k-step s
  __device__ static __forceinline__ int kidx(int s, int grp, int j) { return 32 * s + 16 * (j >> 2) + 4 * grp + (j & 3); }
  // fragment of one row (A) or column (B) stored contiguously along k
  __device__ static __forceinline__ Frag ld(const E* row, int s, int grp) {
    const E* p = row + 32 * s + 4 * grp;
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
    return Frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  __device__ static __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // B operand of k-step s from accumulator tiles (tile t holds contraction rows 16 t ..)
  template <int N>
  __device__ static __forceinline__ Frag from_acc(const f32x4 (&t)[N], int s) {
    Frag f;
    const int t0 = 2 * s, t1 = 2 * s + 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = (__bf16)t[t0][j];
#pragma unroll
    for (int j = 0; j < 4; ++j) f[4 + j] = (t1 < N) ? (__bf16)t[t1 < N ? t1 : 0][j] : (__bf16)0.f;
    return f;
  }
  // scale a fragment elementwise by fp32 factors (slot order)
  __device__ static __forceinline__ Frag scale(Frag f, const float* fac) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (__bf16)((float)f[j] * fac[j]);
    return f;
  }
  static constexpr int SLOTS = 8;
  // number of k-steps covering contraction indices [0, n)
  static constexpr int nks(int n) { return (n + 31) / 32; }
};

// fp32 operands, v_mfma_f32_16x16x4f32
template <>
struct Op<true> {
  using E = float;
  using Frag = float;
  static constexpr int KS = 4;
  __device__ static __forceinline__ int kidx(int s, int grp, int /*j*/) { return 16 * (s >> 2) + 4 * grp + (s & 3); }
  __device__ static __forceinline__ Frag ld(const E* row, int s, int grp) { return row[16 * (s >> 2) + 4 * grp + (s & 3)]; }
  __device__ static __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  template <int N>
  __device__ static __forceinline__ Frag from_acc(const f32x4 (&t)[N], int s) {
    return t[s >> 2][s & 3];
  }
  __device__ static __forceinline__ Frag scale(Frag f, const float* fac) { return f * fac[0]; }
  static constexpr int SLOTS = 1;
  static constexpr int nks(int n) { return n / 4; }
};

// two fp32 -> bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; a in the low half
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// 16x16x16 product D += A B with A given as a[j] = A[lo][4 grp + j] and B as b[j] = B[4 grp + j][lo]
// (accumulator order): one bf16 16x16x16 MFMA, or four fp32 16x16x4 MFMAs.
template <bool F32>
__device__ __forceinline__ f32x4 mma16(const float (&a)[4], const float (&b)[4], f32x4 c) {
  if constexpr (F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  } else {
    const bf16x4 av = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])));
    const bf16x4 bv = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, c, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------------------------
// Packed element stores of operand type E (bf16 or fp32) to LDS or global memory.
// two adjacent elements (4-byte or 8-byte aligned)
template <bool F32>
__device__ __forceinline__ void st2(void* dst, float a, float b) {
  if constexpr (F32) *reinterpret_cast<float2*>(dst) = make_float2(a, b);
  else *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(a, b);
}
// eight adjacent elements (16-byte aligned)
template <bool F32>
__device__ __forceinline__ void st8(void* dst, const float (&x)[8]) {
  if constexpr (F32) {
    float4* d = reinterpret_cast<float4*>(dst);
    d[0] = make_float4(x[0], x[1], x[2], x[3]);
    d[1] = make_float4(x[4], x[5], x[6], x[7]);
  } else {
    *reinterpret_cast<uint4*>(dst) =
        make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
  }
}

// Two adjacent channels of one token, loaded from an fp32 or bf16 tensor (zero when !ok).
template <bool F32>
struct Raw2;
template <>
struct Raw2<false> {
  uint32_t w;
  __device__ __forceinline__ float2 f() const { return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)); }
  __device__ __forceinline__ void load(const void* base, int64_t i, bool ok) {
    w = ok ? *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + i) : 0u;
  }
  // element i (32-bit) of a wave-uniform base: scalar base + vector offset addressing.  The load
  // is unconditional (i must be in bounds); !ok only zeroes the value, so no branch is needed.
  __device__ __forceinline__ void load32(const void* base, uint32_t i, bool ok) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(base) + 2u * i);
    w = ok ? x : 0u;
  }
};
template <>
struct Raw2<true> {
  float2 v;
  __device__ __forceinline__ float2 f() const { return v; }
  __device__ __forceinline__ void load(const void* base, int64_t i, bool ok) {
    v = ok ? *reinterpret_cast<const float2*>(static_cast<const float*>(base) + i) : make_float2(0.f, 0.f);
  }
  __device__ __forceinline__ void load32(const void* base, uint32_t i, bool ok) {
    const float2 x = *reinterpret_cast<const float2*>(static_cast<const char*>(base) + 4u * i);
    v = ok ? x : make_float2(0.f, 0.f);
  }
};

}  // namespace kda
