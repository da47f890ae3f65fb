// KDA chunked backward (training) on gfx950: gradients of L = <dO, o> + <dhT, hT> with respect to
// q, k, v, g, beta and h0, for B equal-length sequences, all on the caller's stream.
//
// The pages give no backward (training with KDA: technical-report page, "Training"); this is the
// chain rule through the chunkwise (UT/WY) forward (architecture blog, "Kimi Delta Attention: the
// linear core").  Per chunk of C tokens from state S0, with G the chunk-local cumulative log-decay,
// Gamma = e^G, gl = G of the last row, L = (I + A)^{-1}, T = L diag(beta), W = T (K Gamma),
// U~ = T V, U = U~ - W S0, P = lowerIncl(Eqk), Kd = K e^{gl - G}:
//
//   1. forward recompute   the forward kernels, keeping the state at every chunk start and the
//                          per-chunk records (-W, Q Gamma, Kd^T, P, U~^T, e^{gl})
//   2. bwd_chain_kernel    the adjoint chain, chunks in reverse, per (sequence, head, 32 value
//                          columns):  dU = P^T dO + Kd dS,  dS <- e^{gl} dS + (Q Gamma)^T dO - W^T dU;
//                          it keeps dS at every chunk end and writes dh0.  It needs no forward state.
//   3. bwd_state_kernel    per (chunk, head), the products with S0 and dS1 (the adjoint at the
//                          chunk's end): U, dU, dP = lowerIncl(dO U^T), d(Q Gamma) = dO S0^T,
//                          dKd = U dS1^T, dW = -dU S0^T, dgl = e^{gl} rowsum(S0 . dS1)
//   4. bwd_intra_kernel    per (chunk, head), through the UT transform: dT = dW (K Gamma)^T + dU V^T,
//                          dV = T^T dU, dL = dT diag(beta), dA = strictLower(-L^T dL L^T), dbeta, and
//                          through Ekk, Eqk (one factor e^{G_r - G_i} <= 1 per (r, i, channel)) and the
//                          elementwise factors into dq, dk, dg (a reverse cumulative sum of dG).
//
// Every product is fp32 arithmetic on operands staged in LDS (bf16 inputs and records stay bf16
// there, which is exact for inputs and is the forward's own operand rounding for records).
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

struct BwdParams {
  const void *q, *k, *v, *g, *beta, *dO;
  const float *h0, *dhT;
  const unsigned char* records;  // one per (chunk, head) item, item = chunk H + head
  // the state after chunk c of head h (full chunks) at item (c H + h), DK DV each, and the adjoint of
  // the state at the end of chunk c of head h at the same item: elements of the operand type (fp32,
  // or bf16 rounded to nearest even -- what the state products round them to anyway)
  const void* states;
  void* dstates;
  float* grads;         // per (chunk, head) item: GradLayout::FLOATS
  void *dq, *dk, *dv, *dg, *dbeta;
  float* dh0;
  int T, H, nch;  // tokens per sequence and chunks per sequence (equal lengths), or T_total and 0
  int units;      // (sequence, head) units: num_seqs H
  int64_t items;  // (chunk, head) items: exact for equal lengths, a bound for packed sequences
  // packed sequences: offsets [num_seqs + 1] and the chunk map of the forward recompute (first chunk
  // of every sequence [num_seqs + 1], the sequences longest first), or NULL
  const int32_t *cu, *chunk0, *order;
  int num_seqs;
  // segments of the adjoint chain (long sequences on few heads): nseg > 1 splits every (sequence,
  // head) into segments of seg_len chunks.  The adjoint chain is affine in the adjoint state at a
  // segment's end, dS_start = N_g dS_end + c_g.  A summary launch writes [c_g | N_g] of segments
  // 1..nseg-1 to bsend slot nseg - 1 - g ([units][nseg - 1][DK][DV + DK]); the combine turns them,
  // from dhT at the last segment's end, into every segment's end adjoint, slot nseg - 1 - g of
  // bstart ([units][nseg][DK][DV]); the main launch then runs every segment from there.
  int nseg, seg_len;
  const float* bstart;
  float* bsend;
};

template <int DK, int DV, int C>
struct GradLayout {
  static constexpr int64_t DU = 0;              // [C][DV]  dU
  static constexpr int64_t DP = DU + C * DV;    // [C][C]   dP, lower-inclusive (zeros above)
  static constexpr int64_t DQG = DP + C * C;    // [C][DK]  d(Q Gamma)
  static constexpr int64_t DKD = DQG + C * DK;  // [C][DK]  dKd
  static constexpr int64_t DW = DKD + C * DK;   // [C][DK]  dW
  static constexpr int64_t DGL = DW + C * DK;   // [DK]     e^{gl} rowsum(S0 . dS1)
  static constexpr int64_t FLOATS = (DGL + DK + 63) & ~(int64_t)63;
};

template <typename E>
__device__ __forceinline__ float tf(E x) {
  return (float)x;
}

// Element i of a wave-uniform base with a 32-bit offset: the access addresses from a scalar base
// plus a 32-bit lane offset instead of forming a 64-bit address in every lane.
template <typename T>
__device__ __forceinline__ T& at(T* base, uint32_t i) {
  return *reinterpret_cast<T*>(reinterpret_cast<unsigned char*>(base) + (uint32_t)sizeof(T) * i);
}
template <typename T>
__device__ __forceinline__ const T& at(const T* base, uint32_t i) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const unsigned char*>(base) + (uint32_t)sizeof(T) * i);
}
// an output element (operand type) at element offset i of a wave-uniform base
template <bool F32>
__device__ __forceinline__ void stg_at(void* base, uint32_t i, float x) {
  if constexpr (F32) at(static_cast<float*>(base), i) = x;
  else at(static_cast<uint16_t*>(base), i) = f32_to_bf16_bits(x);
}

// Token span [a, b) of (sequence, head) unit's sequence n, and its first chunk: equal lengths, or a
// packed sequence with its offsets clamped to [0, T_total] as the forward's chunk map clamps them.
__device__ __forceinline__ void seq_span(const BwdParams& p, int n, int64_t& a, int64_t& b, int64_t& first) {
  if (p.cu) {
    int x = p.cu[n], y = p.cu[n + 1];
    x = x < 0 ? 0 : (x > p.T ? p.T : x);
    y = y < x ? x : (y > p.T ? p.T : y);
    a = x;
    b = y;
    first = p.chunk0[n];
  } else {
    a = (int64_t)n * p.T;
    b = a + p.T;
    first = (int64_t)n * p.nch;
  }
}

// A (chunk, head) item: its head, sequence, first token, length (>= 1), and whether it is the first
// chunk of its sequence
struct BItem {
  int h, seq, len;
  int64_t tok0;
  bool first;
};
template <int C>
__device__ __forceinline__ BItem locate(const BwdParams& p, int64_t item) {
  BItem it;
  const int64_t c = item / p.H;
  it.h = (int)(item - c * p.H);
  int n;
  if (p.cu) {
    int lo = 0, hi = p.num_seqs - 1;  // the last sequence whose first chunk is <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.chunk0[mid] <= c) lo = mid;
      else hi = mid - 1;
    }
    n = lo;
  } else {
    n = (int)(c / p.nch);
  }
  int64_t a, b, first;
  seq_span(p, n, a, b, first);
  it.seq = n;
  it.first = c == first;
  it.tok0 = a + (c - first) * C;
  it.len = (int)min((int64_t)C, b - it.tok0);
  return it;
}
// (chunk, head) items that exist: for packed sequences, counted by the chunk map
__device__ __forceinline__ int64_t item_count(const BwdParams& p) {
  return p.cu ? (int64_t)p.chunk0[p.num_seqs] * p.H : p.items;
}

// acc[i][j] += sum_{k in [k0, k1)} a(i, k) b(k, j)
template <int MI, int NI, typename FA, typename FB>
__device__ __forceinline__ void mac(float (&acc)[MI][NI], int k0, int k1, FA&& a, FB&& b) {
  for (int kk = k0; kk < k1; ++kk) {
    float av[MI], bv[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) av[i] = a(i, kk);
#pragma unroll
    for (int j = 0; j < NI; ++j) bv[j] = b(kk, j);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
}

template <int MI, int NI>
__device__ __forceinline__ void zero(float (&acc)[MI][NI]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = 0.f;
}

// One 16x16 tile of D += A B over the contraction index k in [0, K) on MFMA: a(m, k) and b(k, n)
// (m, n in [0, 16)) give the operand values, rounded to the operand type (bf16 with an fp32
// accumulator, or fp32).  Contraction slots past K read as zero.  In lane (lo, grp) the result is
// acc[r] = D[4 grp + r][lo].
// SPLIT (bf16 only): each operand value x is carried as bf16(x) + bf16(x - bf16(x)) and three
// products are accumulated (hi hi + hi lo + lo hi), for about 16 significant bits where a sum cancels.
// UNR: unroll factor of the contraction loop (fewer registers live at once when small).
template <bool F32, int K, bool SPLIT = false, int UNR = 64, typename FA, typename FB>
__device__ __forceinline__ f32x4 tile_mm(FA&& a, FB&& b, f32x4 acc) {
  using O = Op<F32>;
  const int lane = threadIdx.x & 63, lo = lane & 15, grp = lane >> 4;
#pragma unroll UNR
  for (int s = 0; s < O::nks(K); ++s) {
    typename O::Frag fa, fb, fal, fbl;
    if constexpr (F32) {
      const int k = O::kidx(s, grp, 0);
      fa = a(lo, k);
      fb = b(k, lo);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = O::kidx(s, grp, j);
        const bool ok = (K % 32 == 0) || k < K;
        const float x = ok ? a(lo, k) : 0.f, y = ok ? b(k, lo) : 0.f;
        fa[j] = (__bf16)x;
        fb[j] = (__bf16)y;
        if constexpr (SPLIT) {
          fal[j] = (__bf16)(x - (float)fa[j]);
          fbl[j] = (__bf16)(y - (float)fb[j]);
        }
      }
    }
    acc = O::mma(fa, fb, acc);
    if constexpr (!F32 && SPLIT) {
      acc = O::mma(fa, fbl, acc);
      acc = O::mma(fal, fb, acc);
    }
  }
  return acc;
}

// Two tiles sharing their A operand, D1 += A B1 and D2 += A B2, as tile_mm: A's fragments (and
// their hi + lo split) are formed once for both products.
template <bool F32, int K, bool SPLIT, typename FA, typename FB1, typename FB2>
__device__ __forceinline__ void tile_mm2(FA&& a, FB1&& b1, FB2&& b2, f32x4& d1, f32x4& d2) {
  using O = Op<F32>;
  const int lane = threadIdx.x & 63, lo = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int s = 0; s < O::nks(K); ++s) {
    if constexpr (F32) {
      const int k = O::kidx(s, grp, 0);
      const float fa = a(lo, k);
      d1 = O::mma(fa, b1(k, lo), d1);
      d2 = O::mma(fa, b2(k, lo), d2);
    } else {
      typename O::Frag fa, fal, fb, fbl, fc, fcl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = O::kidx(s, grp, j);
        const bool ok = (K % 32 == 0) || k < K;
        const float x = ok ? a(lo, k) : 0.f, y = ok ? b1(k, lo) : 0.f, z = ok ? b2(k, lo) : 0.f;
        fa[j] = (__bf16)x;
        fb[j] = (__bf16)y;
        fc[j] = (__bf16)z;
        if constexpr (SPLIT) {
          fal[j] = (__bf16)(x - (float)fa[j]);
          fbl[j] = (__bf16)(y - (float)fb[j]);
          fcl[j] = (__bf16)(z - (float)fc[j]);
        }
      }
      d1 = O::mma(fa, fb, d1);
      d2 = O::mma(fa, fc, d2);
      if constexpr (SPLIT) {
        d1 = O::mma(fa, fbl, d1);
        d2 = O::mma(fa, fcl, d2);
        d1 = O::mma(fal, fb, d1);
        d2 = O::mma(fal, fc, d2);
      }
    }
  }
}

// One 16x16 tile of D += A B^T-stored operands read straight from LDS rows that run along the
// contraction index: arow = &A[m0 + lo][0], brow = &Bt[n0 + lo][0] (operand type, 8-byte aligned
// rows for bf16), K a multiple of the MFMA depth.
template <bool F32, int K>
__device__ __forceinline__ f32x4 tile_rows(const typename Op<F32>::E* arow, const typename Op<F32>::E* brow,
                                           f32x4 acc) {
  using O = Op<F32>;
  static_assert(K % O::KS == 0 || F32, "whole MFMA steps");
  const int grp = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int s = 0; s < O::nks(K); ++s) acc = O::mma(O::ld(arow, s, grp), O::ld(brow, s, grp), acc);
  return acc;
}

// Four consecutive elements (operand type) as fp32, from LDS or global memory: one 8-byte (bf16) or
// 16-byte (fp32) access at an aligned address.
template <typename E>
__device__ __forceinline__ float4 ld4f(const E* p) {
  if constexpr (std::is_same<E, float>::value) {
    return *reinterpret_cast<const float4*>(p);
  } else {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
  }
}
__device__ __forceinline__ float4 ld4f(const float4* p) { return *p; }
__device__ __forceinline__ float4 mul4(float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); }
__device__ __forceinline__ float4 exp4(float4 a, float4 b) {  // e^{a - b}
  return make_float4(__expf(a.x - b.x), __expf(a.y - b.y), __expf(a.z - b.z), __expf(a.w - b.w));
}

// tile_mm for operands that run along the contraction index in memory: a4(m, k) returns A[m][k ..
// k + 3] and b4(k, n) returns B[k .. k + 3][n] (k a multiple of 4), so each fragment takes two
// 4-element accesses per operand instead of eight single ones.  K: a multiple of 32 (bf16) or 16 (fp32).
// SPLITB = false with SPLIT: B is exact in bf16 (an input read as it is), so only A is carried as
// hi + lo parts and the hi x lo(B) product, zero, is left out.
template <bool F32, int K, bool SPLIT = false, bool SPLITB = SPLIT, typename FA4, typename FB4>
__device__ __forceinline__ f32x4 tile_mm4(FA4&& a4, FB4&& b4, f32x4 acc) {
  const int lane = threadIdx.x & 63, lo = lane & 15, grp = lane >> 4;
  if constexpr (F32) {
    static_assert(K % 16 == 0, "whole fp32 k-step groups");
    using O = Op<true>;
#pragma unroll
    for (int t = 0; t < K / 16; ++t) {  // k-steps 4 t .. 4 t + 3 take k = 16 t + 4 grp + 0..3
      const float4 x = a4(lo, 16 * t + 4 * grp), y = b4(16 * t + 4 * grp, lo);
      acc = O::mma(x.x, y.x, acc);
      acc = O::mma(x.y, y.y, acc);
      acc = O::mma(x.z, y.z, acc);
      acc = O::mma(x.w, y.w, acc);
    }
  } else {
    static_assert(K % 32 == 0, "whole bf16 k-steps");
    using O = Op<false>;
#pragma unroll
    for (int s = 0; s < K / 32; ++s) {  // slots 0..3: k = 32 s + 4 grp + j, slots 4..7: + 16
      const float4 xa = a4(lo, 32 * s + 4 * grp), xb = a4(lo, 32 * s + 16 + 4 * grp);
      const float4 ya = b4(32 * s + 4 * grp, lo), yb = b4(32 * s + 16 + 4 * grp, lo);
      const float x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
      const float y[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
      typename O::Frag fa, fb, fal, fbl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        fa[j] = (__bf16)x[j];
        fb[j] = (__bf16)y[j];
        if constexpr (SPLIT) fal[j] = (__bf16)(x[j] - (float)fa[j]);
        if constexpr (SPLIT && SPLITB) fbl[j] = (__bf16)(y[j] - (float)fb[j]);
      }
      acc = O::mma(fa, fb, acc);
      if constexpr (SPLIT && SPLITB) acc = O::mma(fa, fbl, acc);
      if constexpr (SPLIT) acc = O::mma(fal, fb, acc);
    }
  }
  return acc;
}

// gfx950's transposing LDS load of 16-bit data: lane L of a 16-lane group points at row k0 + L / 4,
// columns n0 + 4 (L mod 4) of a row-major matrix, and receives column n0 + L at rows k0 .. k0 + 3
// (the lane layout was probed on the GPU).  The address must be 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_tr4(const unsigned char* a) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a));
  return __builtin_bit_cast(bf16x4, x);
}
// bf16 MFMA fragment (A or B) of k-step s for this lane, from an LDS matrix stored with the
// contraction index as its row (row length RL elements, 32 (s + 1) rows at least): column n0 + lo at
// the contraction rows kidx(s, grp, .) = 32 s + 4 grp + 0..3 and 32 s + 16 + 4 grp + 0..3
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* m, int RL, int s, int n0) {
  const int lane = threadIdx.x & 63, lo = lane & 15, grp = lane >> 4;
  const unsigned char* a = reinterpret_cast<const unsigned char*>(m + (32 * s + 4 * grp + (lo >> 2)) * RL + n0 + 4 * (lo & 3));
  const bf16x4 x = lds_tr4(a), y = lds_tr4(a + 32 * RL);
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// ------------------------------------------------------------------------------------------------
// 2. adjoint chain.  One 512-thread workgroup per (sequence, head, 32 value columns), products on
// MFMA.  The record's first four fields (-W, Q Gamma, Kd^T, P) are copied to LDS as stored; dO's
// slice and dU are held in the operand type, the adjoint state dS in fp32 (rounded to the operand
// type only where it is an operand).
template <bool F32, int DK, int DV, int C>
struct BChainCfg {
  using R = Rec<F32, DK, DV, C>;
  using E = typename Op<F32>::E;
  static constexpr int ES = sizeof(E);
  static constexpr int WS = 32, NSL = DV / WS, CP = R::CP, SE = WS + 16 / ES, SS = WS + 4;
  // per buffer: the record prefix (E [R::UT]: -W, Q Gamma, Kd^T, P), e^{gl} (f32 [DK]), dO (E [C][SE])
  static constexpr int REC_BYTES = (int)(R::UT * ES);
  static constexpr int OFF_GAM = REC_BYTES;
  static constexpr int OFF_DO = OFF_GAM + DK * 4;
  static constexpr int BUF = OFF_DO + ((C * SE * ES + 15) & ~15);
  static constexpr int REST = ((C * SE * ES + 15) & ~15) + DK * SS * 4;  // dU (E [C][SE]), dS (f32 [DK][SS])
  // two buffers (the next chunk's record arrives while this one computes) when they fit
  static constexpr bool DBUF = 2 * BUF + REST <= 160 * 1024;
  static constexpr int NBUF = DBUF ? 2 : 1;
  static constexpr int OFF_DU = NBUF * BUF;
  static constexpr int OFF_DS = OFF_DU + ((C * SE * ES + 15) & ~15);
  static constexpr int TOTAL = OFF_DS + DK * SS * 4;
  static constexpr int NTH = 512;
  // dO slice in units of 4 consecutive columns of one row
  static constexpr int N16 = REC_BYTES / 16, NPF = (N16 + NTH - 1) / NTH, NU4 = C * WS / 4, NDO = (NU4 + NTH - 1) / NTH;
  static_assert(REC_BYTES % 16 == 0 && BUF % 16 == 0, "record prefix is a whole number of 16-byte vectors");
  static_assert(DK <= NTH, "one e^{gl} entry per thread");
  static_assert(TOTAL <= 160 * 1024, "LDS");
};

// Registers holding one chunk's record prefix, e^{gl} and dO slice between its load and its store
// into an LDS buffer.
template <bool F32, int DK, int DV, int C>
struct ChainStage {
  using Cf = BChainCfg<F32, DK, DV, C>;
  using R = typename Cf::R;
  using E = typename Cf::E;
  // the slots in one vector each, so that they stay in registers
  typedef uint32_t pf_t __attribute__((ext_vector_type(4 * Cf::NPF)));
  using DW = std::conditional_t<F32, float4, uint2>;  // 4 elements of dO
  pf_t pf;
  float pg;
  DW pdo[Cf::NDO];   // raw dO units: loaded unconditionally (clamped rows), so that no wait for
  bool pok[Cf::NDO];  // them is needed before put; pok: the unit lies in the chunk
  // nodo: the slice is identity columns of a segment summary, whose adjoint has no dO term
  // chunk c (global index) of head h, tokens [tok0, tok0 + nr), nr >= 1
  __device__ __forceinline__ void fetch(const BwdParams& p, int64_t c, int h, int64_t tok0, int nr, int col0, int tid,
                                        bool nodo = false) {
    const unsigned char* rec = p.records + (c * p.H + h) * R::BYTES;
#pragma unroll
    for (int i = 0; i < Cf::NPF; ++i) {
      const int e = tid + Cf::NTH * i;
      const uint4 x = reinterpret_cast<const uint4*>(rec)[e < Cf::N16 ? e : 0];
      pf[4 * i] = x.x;
      pf[4 * i + 1] = x.y;
      pf[4 * i + 2] = x.z;
      pf[4 * i + 3] = x.w;
    }
    pg = reinterpret_cast<const float*>(rec + R::GAM_BYTE)[tid < DK ? tid : 0];
    const int64_t orow = tok0 * p.H + h;
#pragma unroll
    for (int i = 0; i < Cf::NDO; ++i) {
      const int e = tid + Cf::NTH * i, r = (4 * e) / Cf::WS, j = 4 * e - r * Cf::WS;
      const bool ok = !nodo && e < Cf::NU4 && r < nr;  // row 0 always lies in the chunk (nr >= 1)
      pdo[i] = *reinterpret_cast<const DW*>(static_cast<const E*>(p.dO) + (orow + (int64_t)(ok ? r : 0) * p.H) * DV +
                                            (ok ? col0 + j : 0));
      pok[i] = ok;
    }
  }
  __device__ __forceinline__ void put(unsigned char* base, int tid) const {
#pragma unroll
    for (int i = 0; i < Cf::NPF; ++i) {
      const int e = tid + Cf::NTH * i;
      if (e < Cf::N16) reinterpret_cast<uint4*>(base)[e] = make_uint4(pf[4 * i], pf[4 * i + 1], pf[4 * i + 2], pf[4 * i + 3]);
    }
    if (tid < DK) reinterpret_cast<float*>(base + Cf::OFF_GAM)[tid] = pg;
    E* d = reinterpret_cast<E*>(base + Cf::OFF_DO);
#pragma unroll
    for (int i = 0; i < Cf::NDO; ++i) {
      const int e = tid + Cf::NTH * i, r = (4 * e) / Cf::WS, j = 4 * e - r * Cf::WS;
      DW z;
      if constexpr (F32) z = make_float4(0.f, 0.f, 0.f, 0.f);
      else z = make_uint2(0u, 0u);
      if (e < Cf::NU4) *reinterpret_cast<DW*>(d + r * Cf::SE + j) = pok[i] ? pdo[i] : z;
    }
  }
};

// f(e) for e = tid, tid + NTH, ... below N, unrolled with a compile-time trip count (a guarded tail
// only when NTH does not divide N): the loads of every iteration can then be in flight together
// instead of one wait per iteration
template <int N, int NTH, typename F>
__device__ __forceinline__ void for_units(int tid, F&& f) {
#pragma unroll
  for (int i = 0; i < N / NTH; ++i) f(tid + NTH * i);
  if constexpr (N % NTH != 0) {
    if (tid + NTH * (N / NTH) < N) f(tid + NTH * (N / NTH));
  }
}

// Sum over aligned groups of N lanes (N a power of two up to 64), every lane of a group receiving
// the total.  Within 16 lanes the partner values come through DPP (quad permutations for lane xor 1
// and 2, then the mirrors that give lane i lanes 7 - i and 15 - i of its group) rather than through
// an LDS permute; each addition pairs the same two partial sums as a butterfly over xor 1, 2, 4, 8.
template <int CTRL>
__device__ __forceinline__ float dpp_read(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float s) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "lane group");
  if constexpr (N >= 2) s += dpp_read<0xB1>(s);   // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) s += dpp_read<0x4E>(s);   // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) s += dpp_read<0x141>(s);  // row_half_mirror
  if constexpr (N >= 16) s += dpp_read<0x140>(s); // row_mirror
  if constexpr (N >= 32) s += __shfl_xor(s, 16, N);
  if constexpr (N >= 64) s += __shfl_xor(s, 32, N);
  return s;
}

// Eight consecutive elements of an input tensor (element offset i, a multiple of 8) staged in LDS:
// copy8 keeps the element type (bf16 bits or fp32 values unchanged), copy8f widens to fp32.  One
// 16-byte global access per bf16 group (two for fp32); !ok stores zeros.  A select of a loaded
// value on a per-thread condition is compiled into a branch around the load, which then waits on
// its own; staging loops therefore copy every group unconditionally (rows past a sequence's end
// read a valid row) and overwrite those rows with zero8 in a second pass taken only when the chunk
// is short.
template <bool F32>
__device__ __forceinline__ void copy8(const void* src, int64_t i, void* dst, bool ok) {
  if constexpr (F32) {
    const float4* s4 = reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 a = s4[0], b = s4[1];
    reinterpret_cast<float4*>(dst)[0] = ok ? a : z;
    reinterpret_cast<float4*>(dst)[1] = ok ? b : z;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + i);
    *reinterpret_cast<uint4*>(dst) = ok ? w : make_uint4(0u, 0u, 0u, 0u);
  }
}
// copy8 keeping elements 0 .. keep-1 of the group and storing zeros for the rest
template <bool F32>
__device__ __forceinline__ void copy8_head(const void* src, int64_t i, void* dst, int keep) {
  if constexpr (F32) {
    const float4* s4 = reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
    const float4 a = s4[0], b = s4[1];
    reinterpret_cast<float4*>(dst)[0] = make_float4(keep > 0 ? a.x : 0.f, keep > 1 ? a.y : 0.f, keep > 2 ? a.z : 0.f,
                                                    keep > 3 ? a.w : 0.f);
    reinterpret_cast<float4*>(dst)[1] = make_float4(keep > 4 ? b.x : 0.f, keep > 5 ? b.y : 0.f, keep > 6 ? b.z : 0.f,
                                                    keep > 7 ? b.w : 0.f);
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + i);
    auto m = [&](int e) -> uint32_t { return (keep > e ? 0x0000ffffu : 0u) | (keep > e + 1 ? 0xffff0000u : 0u); };
    *reinterpret_cast<uint4*>(dst) = make_uint4(w.x & m(0), w.y & m(2), w.z & m(4), w.w & m(6));
  }
}
// zeros in place of a copy8 group
template <bool F32>
__device__ __forceinline__ void zero8(void* dst) {
  if constexpr (F32) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(dst)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(0u, 0u, 0u, 0u);
  }
}
template <bool F32>
__device__ __forceinline__ void copy8f(const void* src, int64_t i, float* dst, bool ok) {
  if constexpr (F32) {
    copy8<true>(src, i, dst, ok);
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + i);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    float x[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = ok ? __uint_as_float(u[m] << 16) : 0.f;
      x[2 * m + 1] = ok ? __uint_as_float(u[m] & 0xffff0000u) : 0.f;
    }
    reinterpret_cast<float4*>(dst)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// SUM: the summary launch of a segmented adjoint chain (segments 1..nseg-1, d_k more columns that
// start from the identity and see no dO; see BwdParams).
template <bool F32, int DK, int DV, int C, bool SUM>
__global__ __launch_bounds__(512) void bwd_chain_kernel(BwdParams p) {
  using Cf = BChainCfg<F32, DK, DV, C>;
  using R = typename Cf::R;
  using E = typename Cf::E;
  constexpr int WS = Cf::WS, CP = Cf::CP, SE = Cf::SE, SS = Cf::SS;
  constexpr int NSL = (SUM ? DV + DK : DV) / WS;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  E* sdU = reinterpret_cast<E*>(smem + Cf::OFF_DU);
  float* sdS = reinterpret_cast<float*>(smem + Cf::OFF_DS);

  const int tid = threadIdx.x, wave = tid >> 6, lo = tid & 15, grp = (tid >> 4) & 3;
  // Workgroups go to the 8 XCDs round-robin (workgroup i to XCD i mod 8): the value slices of one
  // (sequence, head, segment) are given workgroups 8 apart, so they share one XCD's L2 and each
  // record comes from HBM once.  The grid is padded to a multiple of 8 NSL; padding workgroups exit.
  const int segs = SUM ? p.nseg - 1 : p.nseg;
  const int xcd = blockIdx.x & 7, q8 = blockIdx.x >> 3;
  const int su = (q8 / NSL) * 8 + xcd, col0 = (q8 % NSL) * WS;
  if (su >= p.units * segs) return;
  const int ui = su / segs, g = su - ui * segs + (SUM ? 1 : 0);  // g: the segment
  const int H = p.H;
  // packed sequences are taken longest first (the chunk map's order), so that the long chains start
  // in the first wave of workgroups and the short ones fill in behind them
  const int n = p.order ? p.order[ui / H] : ui / H, h = ui - (ui / H) * H;
  const int unit = n * H + h;
  int64_t t_begin, t_end, first;
  seq_span(p, n, t_begin, t_end, first);
  const int nchu = (int)((t_end - t_begin + C - 1) / C);  // chunks of the sequence
  const int ch_lo = p.nseg > 1 ? g * p.seg_len : 0;
  const int ch_hi = p.nseg > 1 ? min(nchu, (g + 1) * p.seg_len) : nchu;  // chunks [ch_lo, ch_hi), in reverse
  const bool idsl = SUM && col0 >= DV;  // identity columns: no dO term

  // one chunk's record prefix, e^{gl} and dO slice: into registers, then into an LDS buffer
  ChainStage<F32, DK, DV, C> stage;
  auto buf_of = [&](int ch) { return Cf::DBUF ? (ch & 1) : 0; };
  auto fetch_ch = [&](int ch) {  // chunk ch of the sequence
    const int64_t t0 = t_begin + (int64_t)ch * C;
    stage.fetch(p, first + ch, h, t0, (int)min((int64_t)C, t_end - t0), col0, tid, idsl);
  };

  // the adjoint state at the range's end: dhT (or the combine's end adjoint of this segment); a
  // summary starts from zero on the value columns and from the identity on the extra ones
  const float* d_end = p.nseg > 1 ? p.bstart + ((int64_t)unit * p.nseg + (p.nseg - 1 - g)) * DK * DV
                                  : (p.dhT ? p.dhT + (int64_t)unit * DK * DV : nullptr);
  for (int e = tid; e < DK * WS; e += Cf::NTH) {
    const int c = e / WS, j = e - c * WS;
    if constexpr (SUM) sdS[c * SS + j] = (idsl && c == col0 + j - DV) ? 1.f : 0.f;
    else sdS[c * SS + j] = d_end ? d_end[(int64_t)c * DV + col0 + j] : 0.f;
  }
  if (ch_hi > ch_lo) {
    fetch_ch(ch_hi - 1);
    stage.put(smem + buf_of(ch_hi - 1) * Cf::BUF, tid);
  }
  for (int ch = ch_hi - 1; ch >= ch_lo; --ch) {
    __syncthreads();  // this chunk's buffer is filled; dS of the previous step is complete
    if constexpr (!SUM) {
      E* ds_out = static_cast<E*>(p.dstates) + ((first + ch) * H + h) * DK * DV + col0;
      for (int e = tid; e < DK * WS; e += Cf::NTH) {
        const int c = e / WS, j = e - c * WS;
        ds_out[(int64_t)c * DV + j] = (E)sdS[c * SS + j];
      }
    }
    if constexpr (Cf::DBUF) {
      if (ch > ch_lo) fetch_ch(ch - 1);  // in flight while this chunk computes
    }
    const unsigned char* base = smem + buf_of(ch) * Cf::BUF;
    const E* sR = reinterpret_cast<const E*>(base);
    const float* sGam = reinterpret_cast<const float*>(base + Cf::OFF_GAM);
    const E* sdO = reinterpret_cast<const E*>(base + Cf::OFF_DO);
    // dU[i][j] = sum_{r >= i} P[r][i] dO[r][j] + sum_c Kd^T[c][i] dS[c][j]
    // (P is read only where r >= i: its tiles above the diagonal are not all written)
    for (int t = wave; t < (C / 16) * (WS / 16); t += Cf::NTH / 64) {
      const int i0 = 16 * (t / (WS / 16)), j0 = 16 * (t % (WS / 16));
      f32x4 acc = zero4();
      acc = tile_mm<F32, C, false, 1>([&](int m, int k) { return k >= i0 + m ? tf(sR[R::P + k * CP + i0 + m]) : 0.f; },
                            [&](int k, int n) { return tf(sdO[k * SE + j0 + n]); }, acc);
      acc = tile_mm<F32, DK, false, 1>([&](int m, int k) { return tf(sR[R::KPT + k * CP + i0 + m]); },
                             [&](int k, int n) { return sdS[k * SS + j0 + n]; }, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sdU[(i0 + 4 * grp + r) * SE + j0 + lo] = (E)acc[r];
    }
    __syncthreads();
    // dS[c][j] <- e^{gl_c} dS[c][j] + sum_r QG[r][c] dO[r][j] + sum_i (-W)[i][c] dU[i][j]
    for (int t = wave; t < (DK / 16) * (WS / 16); t += Cf::NTH / 64) {
      const int c0 = 16 * (t / (WS / 16)), j0 = 16 * (t % (WS / 16));
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sGam[c0 + 4 * grp + r] * sdS[(c0 + 4 * grp + r) * SS + j0 + lo];
      acc = tile_mm<F32, C, false, 1>([&](int m, int k) { return tf(sR[R::QG + k * DK + c0 + m]); },
                            [&](int k, int n) { return tf(sdO[k * SE + j0 + n]); }, acc);
      acc = tile_mm<F32, C, false, 1>([&](int m, int k) { return tf(sR[R::NW + k * DK + c0 + m]); },
                            [&](int k, int n) { return tf(sdU[k * SE + j0 + n]); }, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sdS[(c0 + 4 * grp + r) * SS + j0 + lo] = acc[r];
    }
    if (ch > ch_lo) {
      if constexpr (Cf::DBUF) {
        stage.put(smem + buf_of(ch - 1) * Cf::BUF, tid);  // the other buffer: last read by the previous step
      } else {
        __syncthreads();  // every read of the one buffer is done
        fetch_ch(ch - 1);
        stage.put(smem, tid);
      }
    }
  }
  __syncthreads();
  if constexpr (SUM) {
    float* se = p.bsend + ((int64_t)unit * (p.nseg - 1) + (p.nseg - 1 - g)) * DK * (DV + DK);
    for (int e = tid; e < DK * WS; e += Cf::NTH) {
      const int c = e / WS, j = e - c * WS;
      se[(int64_t)c * (DV + DK) + col0 + j] = sdS[c * SS + j];
    }
  } else if (p.dh0 && g == 0) {
    for (int e = tid; e < DK * WS; e += Cf::NTH) {
      const int c = e / WS, j = e - c * WS;
      p.dh0[((int64_t)unit * DK + c) * DV + col0 + j] = sdS[c * SS + j];
    }
  }
}

// ------------------------------------------------------------------------------------------------
// 2'. adjoint chain for bf16 records of 32- and 64-token chunks, in the form of the forward chain:
// per (sequence, head, 32 value columns) two chain waves, each holding its 16 columns of dS (fp32)
// in MFMA accumulators across chunks, and four copy waves streaming the next chunk's record prefix
// and dO slice into the other of two LDS buffers.  Every product of the step contracts a record
// field (and dO) over its row index -- dU = P^T dO + K' dS, dS <- e^{gl} dS + (Q Gamma)^T dO +
// (-W)^T dU -- so the fields are staged as stored and their fragments read with the transposing LDS
// load: lane L of a 16-lane group points at row k0 + L / 4, columns n0 + 4 (L mod 4), and receives
// column n0 + L at rows k0 .. k0 + 3.  dS and dU serve as B operands straight from the
// accumulators (no LDS).  Rows are padded by 16 elements, which keeps each half-wave of a
// transposing load on distinct banks.
template <int DK, int DV, int C>
struct BChainTCfg {
  using R = Rec<false, DK, DV, C>;
  static_assert(R::CP == C && C % 32 == 0, "32- or 64-token chunks");
  static constexpr int WS = 32, NCW = 2, NH = 4, NTH = 64 * (NCW + NH), NC = 64 * NH;
  static constexpr int NT = C / 16, KSD = DK / 32, KSC = C / 32;
  static constexpr int RK = DK + 16, RC = C + 16, RW = WS + 16;  // LDS row lengths (elements)
  static constexpr int B_NW = 0;                         // -W       [C][RK]
  static constexpr int B_QG = B_NW + C * RK * 2;         // Q.Gamma  [C][RK]
  static constexpr int B_KPT = B_QG + C * RK * 2;        // K'^T     [DK][RC]
  static constexpr int B_P = B_KPT + DK * RC * 2;        // P        [C][RC]
  static constexpr int B_DO = B_P + C * RC * 2;          // dO slice [C][RW]
  static constexpr int B_GAM = B_DO + C * RW * 2;        // e^{gl}   fp32 [DK]
  static constexpr int BUF = (B_GAM + DK * 4 + 15) & ~15;
  static constexpr int TOTAL = 2 * BUF;
  static_assert(TOTAL <= 163840, "LDS budget of one gfx950 workgroup");
  static_assert(C * WS / 8 <= NC, "one dO unit per copy thread");
};

// one part of a record: NU 16-byte units, UPR per row, from global row stride GROW bytes to LDS row
// stride LROW bytes; loads of units past the end repeat the last one (in bounds), their stores are
// skipped
template <int NC, int NU, int UPR, int GBASE, int GROW, int LBASE, int LROW>
struct TCopy {
  static constexpr int K = (NU + NC - 1) / NC;
  typedef uint32_t vec_t __attribute__((ext_vector_type(4 * K)));
  vec_t st;
  // 32-bit unit offsets formed once and kept in their registers across the chunk loop (the empty
  // asm in load() stops the compiler hoisting them as 64-bit values): each load addresses from the
  // scalar record base, and no offset register is reused as a load destination, which would make
  // the next chunk's loads wait for all of this chunk's
  struct Off {
    uint32_t o[K];
  };
  __device__ static __forceinline__ Off offsets(int ht) {
    Off f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int u = ht + NC * k < NU ? ht + NC * k : NU - 1;
      f.o[k] = (uint32_t)(GBASE + (u / UPR) * GROW + 16 * (u % UPR));
    }
    return f;
  }
  __device__ __forceinline__ void load(const unsigned char* rec, Off& f) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      asm volatile("" : "+v"(f.o[k]));
      const uint4 x = *reinterpret_cast<const uint4*>(rec + f.o[k]);
      st[4 * k] = x.x;
      st[4 * k + 1] = x.y;
      st[4 * k + 2] = x.z;
      st[4 * k + 3] = x.w;
    }
  }
  __device__ __forceinline__ void store(unsigned char* buf, int ht) const {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int u = ht + NC * k;
      if (NU % NC != 0 && u >= NU) continue;
      *reinterpret_cast<uint4*>(buf + LBASE + (u / UPR) * LROW + 16 * (u % UPR)) =
          make_uint4(st[4 * k], st[4 * k + 1], st[4 * k + 2], st[4 * k + 3]);
    }
  }
};

template <int DK, int DV, int C, bool SUM>
__global__ __launch_bounds__(384) void bwd_chain_t_kernel(BwdParams p) {
  using Cf = BChainTCfg<DK, DV, C>;
  using R = typename Cf::R;
  using O = Op<false>;
  using Frag = typename O::Frag;
  constexpr int WS = Cf::WS, NT = Cf::NT, KSD = Cf::KSD, KSC = Cf::KSC;
  constexpr int NSL = (SUM ? DV + DK : DV) / WS;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];

  // (sequence, head, segment, slice) as in bwd_chain_kernel: the slices of one (sequence, head,
  // segment) are workgroups 8 apart, on one XCD
  const int segs = SUM ? p.nseg - 1 : p.nseg;
  const int xcd = blockIdx.x & 7, q8 = blockIdx.x >> 3;
  const int su = (q8 / NSL) * 8 + xcd, col0 = (q8 % NSL) * WS;
  if (su >= p.units * segs) return;
  const int ui = su / segs, g = su - ui * segs + (SUM ? 1 : 0);
  const int H = p.H;
  const int n = p.order ? p.order[ui / H] : ui / H, h = ui - (ui / H) * H;
  const int unit = n * H + h;
  int64_t t_begin, t_end, first;
  seq_span(p, n, t_begin, t_end, first);
  const int nchu = (int)((t_end - t_begin + C - 1) / C);
  const int ch_lo = p.nseg > 1 ? g * p.seg_len : 0;
  const int ch_hi = p.nseg > 1 ? min(nchu, (g + 1) * p.seg_len) : nchu;  // chunks [ch_lo, ch_hi), in reverse
  const int nq = ch_hi > ch_lo ? ch_hi - ch_lo : 0;                      // steps
  const bool idsl = SUM && col0 >= DV;  // identity columns: no dO term

  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wave < Cf::NCW;
  const int wcol = 16 * (chain ? wave : 0);  // this wave's columns within the slice
  const int jc = col0 + wcol + lo;           // this lane's column

  // ---- copy waves: a step's record prefix, e^{gl} and dO slice, global -> registers -> LDS
  auto rec_of = [&](int q) -> const unsigned char* { return p.records + ((first + ch_hi - 1 - q) * H + h) * R::BYTES; };
  struct Stage {
    TCopy<Cf::NC, C * DK / 8, DK / 8, (int)(R::NW * 2), DK * 2, Cf::B_NW, Cf::RK * 2> nw;
    TCopy<Cf::NC, C * DK / 8, DK / 8, (int)(R::QG * 2), DK * 2, Cf::B_QG, Cf::RK * 2> qg;
    TCopy<Cf::NC, DK * C / 8, C / 8, (int)(R::KPT * 2), C * 2, Cf::B_KPT, Cf::RC * 2> kpt;
    TCopy<Cf::NC, C * C / 8, C / 8, (int)(R::P * 2), C * 2, Cf::B_P, Cf::RC * 2> pp;
    TCopy<Cf::NC, DK / 4, DK / 4, (int)R::GAM_BYTE, 0, Cf::B_GAM, 0> gam;
    uint4 dov;
    bool dook;  // the dO unit lies in the chunk (rows past its end, and summary identity columns: zeros)
  };
  const int ht = tid - 64 * Cf::NCW;  // copy-thread index (copy waves only)
  struct Offs {
    typename decltype(Stage::nw)::Off nw;
    typename decltype(Stage::qg)::Off qg;
    typename decltype(Stage::kpt)::Off kpt;
    typename decltype(Stage::pp)::Off pp;
    typename decltype(Stage::gam)::Off gam;
  } offs{decltype(Stage::nw)::offsets(ht), decltype(Stage::qg)::offsets(ht), decltype(Stage::kpt)::offsets(ht),
         decltype(Stage::pp)::offsets(ht), decltype(Stage::gam)::offsets(ht)};
  auto stage_load = [&](Stage& st, int q) {
    const unsigned char* rp = rec_of(q);
    st.nw.load(rp, offs.nw); st.qg.load(rp, offs.qg); st.kpt.load(rp, offs.kpt); st.pp.load(rp, offs.pp);
    st.gam.load(rp, offs.gam);
    // dO: unit ht = (row ht / 4, 8 columns); rows past the chunk's end read its last row (in bounds)
    const int64_t t0 = t_begin + (int64_t)(ch_hi - 1 - q) * C;
    const int len = (int)min((int64_t)C, t_end - t0);
    const int u = ht < C * WS / 8 ? ht : 0, r = u / (WS / 8);
    st.dov = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(p.dO) +
                                             ((t0 + (r < len ? r : len - 1)) * H + h) * DV + col0 + 8 * (u % (WS / 8)));
    st.dook = !idsl && r < len;
  };
  auto stage_store = [&](const Stage& st, unsigned char* b) {
    st.nw.store(b, ht); st.qg.store(b, ht); st.kpt.store(b, ht); st.pp.store(b, ht); st.gam.store(b, ht);
    if (ht < C * WS / 8)
      *reinterpret_cast<uint4*>(b + Cf::B_DO + (ht / (WS / 8)) * Cf::RW * 2 + 16 * (ht % (WS / 8))) =
          st.dook ? st.dov : make_uint4(0u, 0u, 0u, 0u);
  };

  // ---- chain waves: dS[m][r] = dS[16 m + 4 grp + r][jc]
  f32x4 dS[DK / 16];
  // fragment of k-step s of an LDS matrix [rows: contraction][cols: n0 + 0..15], row length RL
  auto frag = [&](const unsigned char* base, int RL, int s, int n0) -> Frag {
    return frag_tr(reinterpret_cast<const __bf16*>(base), RL, s, n0);
  };
  auto step = [&](int q, int buf) {
    const unsigned char* b = smem + buf * Cf::BUF;
    const int ch = ch_hi - 1 - q;
    if (!chain) return;
    if constexpr (!SUM) {  // the adjoint at this chunk's end, as bf16 at the chunk's item slot
      char* ds_out = reinterpret_cast<char*>(static_cast<__bf16*>(p.dstates) + ((first + ch) * H + h) * DK * DV);
      uint32_t z;
      asm volatile("s_mov_b32 %0, 0" : "=s"(z));
      const uint32_t lane_el = (4u * grp + z) * DV + jc;
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<__bf16*>(ds_out + 2u * (lane_el + (uint32_t)(16 * m + r) * DV)) = (__bf16)dS[m][r];
    }
    // dU = K' dS + P^T dO (P^T's k-steps start at the tile's diagonal: the record's P tiles above
    // the diagonal that no step reads are not all written)
    f32x4 dU[NT];
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) dU[bt] = zero4();
#pragma unroll
    for (int sk = 0; sk < KSD; ++sk) {
      const Frag sf = O::from_acc(dS, sk);
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) dU[bt] = O::mma(frag(b + Cf::B_KPT, Cf::RC, sk, 16 * bt), sf, dU[bt]);
    }
    Frag df[KSC];
    if (!idsl) {
#pragma unroll
      for (int s = 0; s < KSC; ++s) df[s] = frag(b + Cf::B_DO, Cf::RW, s, wcol);
#pragma unroll
      for (int bt = 0; bt < NT; ++bt)
#pragma unroll
        for (int s = bt / 2; s < KSC; ++s) dU[bt] = O::mma(frag(b + Cf::B_P, Cf::RC, s, 16 * bt), df[s], dU[bt]);
    }
    // dS <- e^{gl} dS + (Q Gamma)^T dO + (-W)^T dU
    Frag uf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) uf[s] = O::from_acc(dU, s);
    const float* gam = reinterpret_cast<const float*>(b + Cf::B_GAM);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
      const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * m + 4 * grp);
      dS[m][0] *= gm.x;
      dS[m][1] *= gm.y;
      dS[m][2] *= gm.z;
      dS[m][3] *= gm.w;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (!idsl) dS[m] = O::mma(frag(b + Cf::B_QG, Cf::RK, s, 16 * m), df[s], dS[m]);
        dS[m] = O::mma(frag(b + Cf::B_NW, Cf::RK, s, 16 * m), uf[s], dS[m]);
      }
    }
  };

  if (chain) {
    // the adjoint at the range's end: dhT (or the combine's end adjoint of this segment); a summary
    // starts from zero on the value columns and from the identity on the extra ones
    const float* d_end = p.nseg > 1 ? p.bstart + ((int64_t)unit * p.nseg + (p.nseg - 1 - g)) * DK * DV
                                    : (p.dhT ? p.dhT + (int64_t)unit * DK * DV : nullptr);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * m + 4 * grp + r;
        if constexpr (SUM) dS[m][r] = (idsl && c == jc - DV) ? 1.f : 0.f;
        else dS[m][r] = d_end ? d_end[(int64_t)c * DV + jc] : 0.f;
      }
    __syncthreads();
    for (int q = 0; q < nq; q += 2) {
      step(q, 0);
      __syncthreads();
      if (q + 1 >= nq) break;
      step(q + 1, 1);
      __syncthreads();
    }
    if constexpr (SUM) {
      float* se = p.bsend + ((int64_t)unit * (p.nseg - 1) + (p.nseg - 1 - g)) * DK * (DV + DK);
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) se[(int64_t)(16 * m + 4 * grp + r) * (DV + DK) + jc] = dS[m][r];
    } else if (p.dh0 && g == 0) {
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) p.dh0[((int64_t)unit * DK + 16 * m + 4 * grp + r) * DV + jc] = dS[m][r];
    }
  } else {
    // invariant at step q: buffer q & 1 holds step q, stage (q + 1) & 1 holds step q + 1; steps past
    // the last are clamped to it (copies into a buffer nobody reads)
    Stage s0, s1;
    const int last = nq - 1;
    if (nq > 0) {
      stage_load(s0, 0);
      stage_store(s0, smem);
      stage_load(s1, last < 1 ? last : 1);
    }
    __syncthreads();
    for (int q = 0; q < nq; q += 2) {
      stage_load(s0, q + 2 < last ? q + 2 : last);
      stage_store(s1, smem + Cf::BUF);
      __syncthreads();
      if (q + 1 >= nq) break;
      stage_load(s1, q + 3 < last ? q + 3 : last);
      stage_store(s0, smem);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------------------------
// 3. products with the chunk's start state S0 and end adjoint dS1, one 512-thread workgroup per
// (chunk, head), on MFMA.  S0, dS1, dO, U and dU are staged in LDS in the operand type (rows padded
// by 16 bytes); the record's -W, then P (masked to its lower triangle) and Kd^T, share one region.
template <bool F32, int DK, int DV, int C, int VP_>
struct BStateLayout {
  using E = typename Op<F32>::E;
  static constexpr int ES = sizeof(E);
  // row padding: 16 bytes where the rows are also read straight along a row (16 rows of one 8-byte
  // access each then fall on distinct banks), 32 bytes for P and Kd^T, read only with the transposing
  // load (whose half-wave covers 8 consecutive rows)
  static constexpr int SV = VP_ + 16 / ES, SK = DK + 16 / ES, SC = C + 32 / ES;
  static constexpr int OFF_S0 = 0;                                  // E [DK][SV]
  static constexpr int OFF_DS = OFF_S0 + DK * SV * ES;              // E [DK][SV]
  static constexpr int OFF_DO = OFF_DS + DK * SV * ES;              // E [C][SV]
  static constexpr int OFF_U = OFF_DO + C * SV * ES;                // E [C][SV]
  static constexpr int OFF_DU = OFF_U + C * SV * ES;                // E [C][SV]
  static constexpr int OFF_X = OFF_DU + C * SV * ES;                // E: -W [C][SK], then P [C][SC] + Kd^T [DK][SC]
  static constexpr int X_BYTES = (C * SK > (C + DK) * SC ? C * SK : (C + DK) * SC) * ES;
  static constexpr int TOTAL = OFF_X + X_BYTES;
};
// The value columns are taken VP at a time (all of them where the LDS holds them, else halves or
// quarters): U and dU are per column, and the other products sum over the columns, so a pass adds
// its share to them.
template <bool F32, int DK, int DV, int C>
struct BStateCfg {
  using R = Rec<F32, DK, DV, C>;
  using E = typename Op<F32>::E;
  using GL = GradLayout<DK, DV, C>;
  static constexpr int NTH = 512;
  static constexpr int VP = BStateLayout<F32, DK, DV, C, DV>::TOTAL <= 160 * 1024       ? DV
                            : BStateLayout<F32, DK, DV, C, DV / 2>::TOTAL <= 160 * 1024 ? DV / 2
                                                                                          : DV / 4;
  using L = BStateLayout<F32, DK, DV, C, VP>;
  static constexpr int SV = L::SV, SK = L::SK, SC = L::SC;
  static constexpr int OFF_S0 = L::OFF_S0, OFF_DS = L::OFF_DS, OFF_DO = L::OFF_DO, OFF_U = L::OFF_U,
                       OFF_DU = L::OFF_DU, OFF_X = L::OFF_X, TOTAL = L::TOTAL;
  static_assert(OFF_X % 16 == 0, "alignment");
  static_assert(TOTAL <= 160 * 1024, "LDS");
  static_assert(VP % 16 == 0, "whole 16-column tiles per pass");
};

template <bool F32, int DK, int DV, int C>
__global__ __launch_bounds__(512) void bwd_state_kernel(BwdParams p) {
  using Cf = BStateCfg<F32, DK, DV, C>;
  using R = typename Cf::R;
  using E = typename Cf::E;
  using GL = typename Cf::GL;
  constexpr int SV = Cf::SV, SK = Cf::SK, SC = Cf::SC, CP = R::CP, NTH = Cf::NTH, VP = Cf::VP;
  // bf16 with 32- or 64-token chunks: the products read whole MFMA fragments (the transposing LDS
  // load where the contraction runs along a matrix's rows) instead of building them element by element
  constexpr bool TRF = !F32 && C % 32 == 0;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  E* sS0 = reinterpret_cast<E*>(smem + Cf::OFF_S0);
  E* sdS = reinterpret_cast<E*>(smem + Cf::OFF_DS);
  E* sdO = reinterpret_cast<E*>(smem + Cf::OFF_DO);
  E* sU = reinterpret_cast<E*>(smem + Cf::OFF_U);
  E* sdU = reinterpret_cast<E*>(smem + Cf::OFF_DU);
  E* sNW = reinterpret_cast<E*>(smem + Cf::OFF_X);
  E* sP = reinterpret_cast<E*>(smem + Cf::OFF_X);
  E* sKPT = sP + C * SC;

  const int64_t item = blockIdx.x;
  if (item >= item_count(p)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lo = tid & 15, grp = (tid >> 4) & 3, H = p.H;
  const BItem it = locate<C>(p, item);
  const int h = it.h, nr = it.len;
  const int64_t unit = (int64_t)it.seq * H + h;
  const E* rec = reinterpret_cast<const E*>(p.records + item * R::BYTES);
  const float* gam = reinterpret_cast<const float*>(p.records + item * R::BYTES + R::GAM_BYTE);
  // the chunk's start state: the state after the sequence's previous chunk (item - H, operand type),
  // or h0 (fp32) for a sequence's first chunk, or zero
  const E* s0c = !it.first ? static_cast<const E*>(p.states) + (item - H) * DK * DV : nullptr;
  const float* s0h = it.first && p.h0 ? p.h0 + unit * DK * DV : nullptr;
  const E* ds1 = static_cast<const E*>(p.dstates) + item * DK * DV;
  float* gr = p.grads + item * GL::FLOATS;
  const int64_t orow = it.tok0 * H + h;

#pragma unroll
  for (int vp0 = 0; vp0 < DV; vp0 += VP) {
    // a sum over the value columns: the first pass writes it, later ones add their share (each
    // element has one owner thread in every pass)
    auto put = [&](uint32_t i, float x) { at(gr, i) = vp0 == 0 ? x : at(gr, i) + x; };
    if (vp0 > 0) __syncthreads();  // the previous pass's reads of every LDS region are done
    // columns [vp0, vp0 + VP) of S0 and dS1 to LDS, 4 elements per access; the source of S0 (a kept
    // state, h0, or none: zeros) is chosen once for the workgroup, so no load sits under a
    // per-element select
    auto stage_states = [&](auto s0_kind) {
      constexpr int K = decltype(s0_kind)::value;  // 0 none, 1 kept state, 2 h0
      for_units<DK * VP / 4, NTH>(tid, [&](int e) {
        const int c = (4 * e) / VP, j = 4 * e - c * VP;
        const int64_t gi = (int64_t)c * DV + vp0 + j;
        E* pa = sS0 + c * SV + j;
        E* pd = sdS + c * SV + j;
        if constexpr (F32) {
          float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
          if constexpr (K == 1) a = *reinterpret_cast<const float4*>(s0c + gi);
          if constexpr (K == 2) a = *reinterpret_cast<const float4*>(s0h + gi);
          const float4 d = *reinterpret_cast<const float4*>(ds1 + gi);
          pa[0] = a.x; pa[1] = a.y; pa[2] = a.z; pa[3] = a.w;
          pd[0] = d.x; pd[1] = d.y; pd[2] = d.z; pd[3] = d.w;
        } else {
          bf16x4 a = {(E)0.f, (E)0.f, (E)0.f, (E)0.f};
          if constexpr (K == 1) a = *reinterpret_cast<const bf16x4*>(s0c + gi);
          if constexpr (K == 2) {
            const float4 x = *reinterpret_cast<const float4*>(s0h + gi);
            a = bf16x4{(E)x.x, (E)x.y, (E)x.z, (E)x.w};
          }
          const bf16x4 d = *reinterpret_cast<const bf16x4*>(ds1 + gi);
          *reinterpret_cast<bf16x4*>(pa) = a;
          *reinterpret_cast<bf16x4*>(pd) = d;
        }
      });
    };
    if (s0c)
      stage_states(std::integral_constant<int, 1>{});
    else if (s0h)
      stage_states(std::integral_constant<int, 2>{});
    else
      stage_states(std::integral_constant<int, 0>{});
    for_units<C * VP / 8, NTH>(tid, [&](int e) {
      const int r = (8 * e) / VP, j = 8 * e - r * VP;
      copy8<F32>(p.dO, (orow + (int64_t)(r < nr ? r : 0) * H) * DV + vp0 + j, sdO + r * SV + j, true);
    });
    for_units<C * DK / 8, NTH>(tid, [&](int e) {
      const int r = (8 * e) / DK, c = 8 * e - r * DK;
      copy8<F32>(rec, R::NW + 8 * e, sNW + r * SK + c, true);
    });
    if (nr < C) {  // the same threads overwrite dO's rows past the end with zeros
      for_units<C * VP / 8, NTH>(tid, [&](int e) {
        const int r = (8 * e) / VP, j = 8 * e - r * VP;
        if (r >= nr) zero8<F32>(sdO + r * SV + j);
      });
    }
    __syncthreads();
    // U = U~ + (-W) S0  (U~ from the record's U~^T)
    for (int t = wave; t < (C / 16) * (VP / 16); t += NTH / 64) {
      const int i0 = 16 * (t / (VP / 16)), j0 = 16 * (t % (VP / 16));
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = tf(rec[R::UT + (vp0 + j0 + lo) * C + i0 + 4 * grp + r]);
      if constexpr (TRF) {  // -W rows run along the contraction; S0 is read with the transposing load
#pragma unroll
        for (int sk = 0; sk < DK / 32; ++sk)
          acc = Op<false>::mma(Op<false>::ld(sNW + (i0 + lo) * SK, sk, grp), frag_tr(sS0, SV, sk, j0), acc);
      } else {
        acc = tile_mm<F32, DK>([&](int m, int k) { return tf(sNW[(i0 + m) * SK + k]); },
                               [&](int k, int n) { return tf(sS0[k * SV + j0 + n]); }, acc);  // S0 runs along n
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sU[(i0 + 4 * grp + r) * SV + j0 + lo] = (E)acc[r];
    }
    // e^{gl} rowsum(S0 . dS1): NTH / DK adjacent lanes per channel, each over every (NTH / DK)-th column
    {
      constexpr int NPCH = NTH / DK;
      static_assert(NPCH * DK == NTH && (NPCH & (NPCH - 1)) == 0 && NPCH <= 64, "lanes per channel");
      const int c = tid / NPCH, part = tid - c * NPCH;
      float sum = 0.f;
      for (int j = part; j < VP; j += NPCH) sum = fmaf(tf(sS0[c * SV + j]), tf(sdS[c * SV + j]), sum);
#pragma unroll
      for (int off = 1; off < NPCH; off <<= 1) sum += __shfl_xor(sum, off);
      if (part == 0) put(GL::DGL + c, gam[c] * sum);
    }
    __syncthreads();
    for_units<C * C / 8, NTH>(tid, [&](int e) {  // P's lower triangle (record tiles above it are not all written)
      const int s_ = (8 * e) / C, r = 8 * e - s_ * C;
      copy8_head<F32>(rec, R::P + s_ * CP + r, sP + s_ * SC + r, s_ - r + 1);
    });
    for_units<DK * C / 8, NTH>(tid, [&](int e) {
      const int c = (8 * e) / C, r = 8 * e - c * C;
      copy8<F32>(rec, R::KPT + c * CP + r, sKPT + c * SC + r, true);
    });
    __syncthreads();
    // dU[r][j] = sum_{s >= r} P[s][r] dO[s][j] + sum_c Kd^T[c][r] dS1[c][j]
    for (int t = wave; t < (C / 16) * (VP / 16); t += NTH / 64) {
      const int i0 = 16 * (t / (VP / 16)), j0 = 16 * (t % (VP / 16));
      f32x4 acc = zero4();
      if constexpr (TRF) {  // P^T, dO, Kd and dS1 all contract over their rows: transposing loads
#pragma unroll
        for (int sk = 0; sk < C / 32; ++sk) acc = Op<false>::mma(frag_tr(sP, SC, sk, i0), frag_tr(sdO, SV, sk, j0), acc);
#pragma unroll
        for (int sk = 0; sk < DK / 32; ++sk)
          acc = Op<false>::mma(frag_tr(sKPT, SC, sk, i0), frag_tr(sdS, SV, sk, j0), acc);
      } else {
        acc = tile_mm<F32, C>([&](int m, int k) { return tf(sP[k * SC + i0 + m]); },
                              [&](int k, int n) { return tf(sdO[k * SV + j0 + n]); }, acc);
        acc = tile_mm<F32, DK>([&](int m, int k) { return tf(sKPT[k * SC + i0 + m]); },
                               [&](int k, int n) { return tf(sdS[k * SV + j0 + n]); }, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sdU[(i0 + 4 * grp + r) * SV + j0 + lo] = (E)acc[r];
        at(gr, GL::DU + (i0 + 4 * grp + r) * DV + vp0 + j0 + lo) = acc[r];
      }
    }
    __syncthreads();
    // dP = lowerIncl(dO U^T)
    for (int t = wave; t < (C / 16) * (C / 16); t += NTH / 64) {
      const int i0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
      f32x4 acc = zero4();
      if (n0 <= i0) acc = tile_rows<F32, VP>(sdO + (i0 + lo) * SV, sU + (n0 + lo) * SV, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = i0 + 4 * grp + r, col = n0 + lo;
        put(GL::DP + row * C + col, col <= row ? acc[r] : 0.f);
      }
    }
    // d(Q Gamma) = dO S0^T, dKd = U dS1^T, dW = -dU S0^T
    for (int t = wave; t < 3 * (C / 16) * (DK / 16); t += NTH / 64) {
      const int which = t / ((C / 16) * (DK / 16)), tt = t - which * ((C / 16) * (DK / 16));
      const int i0 = 16 * (tt / (DK / 16)), c0 = 16 * (tt % (DK / 16));
      const E* A = which == 0 ? sdO : which == 1 ? sU : sdU;
      const E* Bt = which == 1 ? sdS : sS0;
      f32x4 acc = tile_rows<F32, VP>(A + (i0 + lo) * SV, Bt + (c0 + lo) * SV, zero4());
      const int64_t off = which == 0 ? GL::DQG : which == 1 ? GL::DKD : GL::DW;
      const float sg = which == 2 ? -1.f : 1.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) put(off + (i0 + 4 * grp + r) * DK + c0 + lo, sg * acc[r]);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// 4. through the UT transform, one 512-thread workgroup per (chunk, head).  [C][DK] results live in
// MFMA accumulator tiles: wave w owns tiles w + 8 q of the (C/16) x (DK/16) grid.  Exponent
// differences are taken against a per-16-row-tile reference so that every factor is finite in fp32
// at g >= -5: for a row tile, R = G just before it (row factors e^{G_r - R} in [e^{-80}, 1], column
// factors e^{R - G_i} <= e^{80} for i in the tile and <= 1 before it); for a column tile, R' = G at
// its last row (the mirror image).
template <bool F32, int DK, int DV, int C>
struct BIntraCfg {
  using E = typename Op<F32>::E;
  static constexpr int NTH = 512, ES = sizeof(E);
  static constexpr int NTC = C / 16, NTK = DK / 16, NTV = DV / 16;
  static constexpr int NTILE = NTC * NTK, MAXT = (NTILE + 7) / 8, NPAIR = NTC * (NTC + 1) / 2;
  static constexpr int NPART = NTH / DK, RPP = C / NPART;       // scans: row parts per channel
  static constexpr int SG = DK + 4, SK = DK + 16 / ES, SV = DV + 16 / ES, SM = C + 4;
  // q and v staged in LDS where they fit beside the rest (fp32 at d_k = 128, chunk 64: read from
  // global memory where they are used instead)
  static constexpr int REST = C * SG * 4 + C * SK * ES + 4 * C * SM * 4 + 2 * C * 4 + (C / 16 + NPART + 1) * DK * 4;
  static constexpr bool QV_LDS = REST + C * SK * ES + C * SV * ES <= 160 * 1024;
  static constexpr int OFF_G = 0;                                // f32 [C][SG]  g, G, then dG
  static constexpr int OFF_K = OFF_G + C * SG * 4;               // E [C][SK]
  static constexpr int OFF_Q = OFF_K + C * SK * ES;              // E [C][SK] (QV_LDS)
  static constexpr int OFF_V = OFF_Q + (QV_LDS ? C * SK * ES : 0);       // E [C][SV] (QV_LDS)
  static constexpr int OFF_EKK = OFF_V + (QV_LDS ? C * SV * ES : 0);     // f32 [C][SM] Ekk (strict lower)
  static constexpr int OFF_L = OFF_EKK + C * SM * 4;             // f32 [C][SM] L = (I + A)^{-1}
  static constexpr int OFF_M3 = OFF_L + C * SM * 4;              // f32 [C][SM] dT -> dL -> dA -> dEkk
  static constexpr int OFF_M4 = OFF_M3 + C * SM * 4;             // f32 [C][SM] L^T dL, then dEqk
  static constexpr int OFF_BETA = OFF_M4 + C * SM * 4;           // f32 [C]
  static constexpr int OFF_DB = OFF_BETA + C * 4;                // f32 [C]
  static constexpr int OFF_RED = OFF_DB + C * 4;                 // f32 [NTC][DK]
  static constexpr int OFF_SCAN = OFF_RED + NTC * DK * 4;        // f32 [NPART][DK]
  static constexpr int OFF_DGL = OFF_SCAN + NPART * DK * 4;      // f32 [DK]
  static constexpr int TOTAL = OFF_DGL + DK * 4;
  static_assert(NPART * DK == NTH && RPP * NPART == C && 64 * NTC <= NTH, "thread layout");
  static_assert((C * SK * ES) % 16 == 0 && (C * SV * ES) % 16 == 0, "alignment");
  static_assert(TOTAL <= 160 * 1024, "LDS");
  static_assert(TOTAL == REST + (QV_LDS ? C * SK * ES + C * SV * ES : 0), "layout");
};

// (b, a) of the a-th ... pair index t over the lower triangle of tiles, a <= b
__device__ __forceinline__ void tri_pair(int t, int& b, int& a) {
  b = 0;
  while (t > b) {
    t -= b + 1;
    ++b;
  }
  a = t;
}

// Inclusive prefix sums down the rows of an LDS [C][ld] fp32 array, per channel, in place (reverse:
// suffix sums).  Thread (channel tid % DK, part tid / DK) scans RPP rows; the parts' totals go
// through `tot` [NPART][DK].
template <int DK, int C, int NPART, int RPP, bool REV>
__device__ __forceinline__ void scan_rows(float* a, int ld, float* tot, int tid) {
  const int c = tid % DK, part = tid / DK;
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < RPP; ++u) {
    const int r = REV ? C - 1 - (part * RPP + u) : part * RPP + u;
    s += a[r * ld + c];
    a[r * ld + c] = s;
  }
  tot[part * DK + c] = s;
  __syncthreads();
  float off = 0.f;
  for (int q = 0; q < part; ++q) off += tot[q * DK + c];
#pragma unroll
  for (int u = 0; u < RPP; ++u) {
    const int r = REV ? C - 1 - (part * RPP + u) : part * RPP + u;
    a[r * ld + c] += off;
  }
  __syncthreads();
}

// Rows 0 .. nr-1 of a bf16 [C][D + 8] LDS tile to an output whose row r starts D * H * r elements
// after `base`: 16-byte accesses, 8 elements each, so every row of the output (D * 2 contiguous
// bytes) is written as whole 64-byte pieces rather than 2-byte elements.
template <int C, int D, int NTH>
__device__ __forceinline__ void rows_out_bf16(const __bf16* src, void* base, int H, int nr, int tid) {
  for_units<C * D / 8, NTH>(tid, [&](int e) {
    const int r = (8 * e) / D, c = 8 * e - r * D;
    if (r < nr)
      at(static_cast<uint4*>(base), (uint32_t)((r * H * D + c) / 8)) =
          *reinterpret_cast<const uint4*>(src + r * (D + 8) + c);
  });
}

template <bool F32, int DK, int DV, int C>
__global__ __launch_bounds__(512) void bwd_intra_kernel(BwdParams p) {
  using Cf = BIntraCfg<F32, DK, DV, C>;
  using E = typename Cf::E;
  using GL = GradLayout<DK, DV, C>;
  constexpr int NTK = Cf::NTK, NTV = Cf::NTV, NTILE = Cf::NTILE, MAXT = Cf::MAXT;
  // owned tile q of this wave, t = wave + 8 q of the (C/16) x (DK/16) grid: its row tile and channel
  // tile.  At d_k = 128 (8 channel tiles) the row tile is q itself, known at compile time in the
  // unrolled loops over q, so the loops over its rows get constant trip counts and offsets.
  auto tile_row = [&](int q, int t) { return NTK == 8 ? q : t / NTK; };
  auto tile_col = [&](int t) { return NTK == 8 ? (t & 7) : t % NTK; };
  constexpr int EEU = NTK == 8 ? C / 4 : 1;  // unrolling of the loops over a row tile's rows (constant counts at d_k = 128)
  constexpr int SG = Cf::SG, SK = Cf::SK, SV = Cf::SV, SM = Cf::SM, NTH = Cf::NTH;
  // bf16 gradients staged in LDS regions that are dead by then and written out as whole rows: dv in
  // M4 (free until Y), dq and dk over Ekk and L (free after dA), where a [C][d + 8] tile fits
  constexpr bool STG_V = !F32 && C * (DV + 8) * 2 <= C * SM * 4;
  constexpr bool STG_QK = !F32 && C * (DK + 8) * 2 <= C * SM * 4;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  float* sG = reinterpret_cast<float*>(smem + Cf::OFF_G);
  E* sK = reinterpret_cast<E*>(smem + Cf::OFF_K);
  E* sQ = reinterpret_cast<E*>(smem + Cf::OFF_Q);
  E* sV = reinterpret_cast<E*>(smem + Cf::OFF_V);
  float* sEkk = reinterpret_cast<float*>(smem + Cf::OFF_EKK);
  float* sL = reinterpret_cast<float*>(smem + Cf::OFF_L);
  float* sM3 = reinterpret_cast<float*>(smem + Cf::OFF_M3);
  float* sM4 = reinterpret_cast<float*>(smem + Cf::OFF_M4);
  float* sBeta = reinterpret_cast<float*>(smem + Cf::OFF_BETA);
  float* sDb = reinterpret_cast<float*>(smem + Cf::OFF_DB);
  float* sRed = reinterpret_cast<float*>(smem + Cf::OFF_RED);
  float* sScan = reinterpret_cast<float*>(smem + Cf::OFF_SCAN);
  float* sDgl = reinterpret_cast<float*>(smem + Cf::OFF_DGL);

  const int64_t item = blockIdx.x;
  if (item >= item_count(p)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lo = tid & 15, grp = (tid >> 4) & 3, H = p.H;
  const BItem it = locate<C>(p, item);
  const int h = it.h, nr = it.len;
  const int64_t row0 = it.tok0 * H + h;  // (token, head) row of the chunk's first token
  // wave-uniform bases of the chunk's rows in the outputs (32-bit element offsets from them)
  constexpr int ES_ = F32 ? 4 : 2;
  void* dqb = static_cast<unsigned char*>(p.dq) + row0 * DK * ES_;
  void* dkb = static_cast<unsigned char*>(p.dk) + row0 * DK * ES_;
  void* dgb = static_cast<unsigned char*>(p.dg) + row0 * DK * ES_;
  void* dvb = static_cast<unsigned char*>(p.dv) + row0 * DV * ES_;
  void* dbb = static_cast<unsigned char*>(p.dbeta) + row0 * ES_;
  const float* gr = p.grads + item * GL::FLOATS;

  // ---- stage q, k, v, g, beta, 8 consecutive channels per access (rows past the chunk's end read
  // row 0 and store zeros), then G = cumsum(g)
  for_units<C * DK / 8, NTH>(tid, [&](int e) {
    const int r = (8 * e) / DK, c = 8 * e - r * DK;
    const bool ok = r < nr;
    const int64_t gi = (row0 + (int64_t)(ok ? r : 0) * H) * DK + c;
    if constexpr (Cf::QV_LDS) copy8<F32>(p.q, gi, sQ + r * SK + c, true);
    copy8<F32>(p.k, gi, sK + r * SK + c, true);
    copy8f<F32>(p.g, gi, sG + r * SG + c, ok);
  });
  if constexpr (Cf::QV_LDS) {
    for_units<C * DV / 8, NTH>(tid, [&](int e) {
      const int r = (8 * e) / DV, j = 8 * e - r * DV;
      copy8<F32>(p.v, (row0 + (int64_t)(r < nr ? r : 0) * H) * DV + j, sV + r * SV + j, true);
    });
  }
  if (nr < C) {  // the same threads overwrite the rows past the end with zeros
    for_units<C * DK / 8, NTH>(tid, [&](int e) {
      const int r = (8 * e) / DK, c = 8 * e - r * DK;
      if (r >= nr) {
        if constexpr (Cf::QV_LDS) zero8<F32>(sQ + r * SK + c);
        zero8<F32>(sK + r * SK + c);
      }
    });
    if constexpr (Cf::QV_LDS) {
      for_units<C * DV / 8, NTH>(tid, [&](int e) {
        const int r = (8 * e) / DV, j = 8 * e - r * DV;
        if (r >= nr) zero8<F32>(sV + r * SV + j);
      });
    }
  }
  // q[r][c] and v[r][j .. j + 3] of the chunk (zero past its end): from LDS, or from global memory
  auto q_at = [&](int r, int c) -> float {
    if constexpr (Cf::QV_LDS) return tf(sQ[r * SK + c]);
    else return r < nr ? ldg<F32>(p.q, (row0 + (int64_t)r * H) * DK + c) : 0.f;
  };
  auto v4_at = [&](int r, int j) -> float4 {  // v[r][j .. j + 3], j a multiple of 4
    if constexpr (Cf::QV_LDS) {
      return ld4f(sV + r * SV + j);
    } else {
      const float4 x = ld4f(static_cast<const E*>(p.v) + (row0 + (int64_t)(r < nr ? r : 0) * H) * DV + j);
      return r < nr ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (tid < C) sBeta[tid] = tid < nr ? ldg<F32>(p.beta, row0 + (int64_t)tid * H) : 0.f;
  __syncthreads();
  scan_rows<DK, C, Cf::NPART, Cf::RPP, false>(sG, SG, sScan, tid);

  // ---- Ekk = strictLower(K e^{G - R_b}) (K e^{R_b - G})^T per tile pair (b, a), a <= b
  for (int t = wave; t < Cf::NPAIR; t += 8) {
    int tb, ta;
    tri_pair(t, tb, ta);
    const int r0 = 16 * tb, i0 = 16 * ta;
    const float* Rb = tb > 0 ? sG + (r0 - 1) * SG : nullptr;
    auto rb4 = [&](int k) { return Rb ? *reinterpret_cast<const float4*>(Rb + k) : make_float4(0.f, 0.f, 0.f, 0.f); };
    auto g4 = [&](int r, int k) { return *reinterpret_cast<const float4*>(sG + r * SG + k); };
    f32x4 acc = tile_mm4<F32, DK>(
        [&](int m, int k) { return mul4(ld4f(sK + (r0 + m) * SK + k), exp4(g4(r0 + m, k), rb4(k))); },
        [&](int k, int n) { return mul4(ld4f(sK + (i0 + n) * SK + k), exp4(rb4(k), g4(i0 + n, k))); }, zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * grp + r, col = i0 + lo;
      sEkk[row * SM + col] = col < row ? acc[r] : 0.f;
    }
  }
  for (int e = tid; e < C * C; e += NTH) {
    const int r = e / C, i = e - r * C;
    if ((i >> 4) > (r >> 4)) sEkk[r * SM + i] = 0.f;
  }
  __syncthreads();

  // ---- L = (I + A)^{-1}, A = diag(beta) Ekk (strictly lower), in 16x16 blocks: the diagonal blocks
  // by forward substitution, one wave each (one column per lane); then, one wave per column block a,
  // the blocks below it in order, L_ba = -L_bb sum_{c=a}^{b-1} A_bc L_ca, on fp32 MFMA -- 16
  // dependent substitution steps instead of C.  Blocks above the diagonal are zero.
  constexpr int NTC = Cf::NTC;
  if (wave < NTC) {
    const int b = wave, j = lo;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* arow = sEkk + (16 * b + r) * SM + 16 * b;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s = fmaf(arow[i], x[i], s);
      x[r] = (r == j ? 1.f : 0.f) - sBeta[16 * b + r] * s;
    }
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sL[(16 * b + r) * SM + 16 * b + j] = x[r];
    }
  } else {
    for (int e = tid - 64 * NTC; e < C * C; e += NTH - 64 * NTC) {
      const int r = e / C, i = e - r * C;
      if ((i >> 4) > (r >> 4)) sL[r * SM + i] = 0.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a + 1 < NTC; ++a) {
    if (wave != a) continue;
    float Xb[NTC][4];  // Xb[c][r] = L_ca[4 grp + r][lo] (accumulator order)
#pragma unroll
    for (int r = 0; r < 4; ++r) Xb[a][r] = sL[(16 * a + 4 * grp + r) * SM + 16 * a + lo];
#pragma unroll
    for (int b = a + 1; b < NTC; ++b) {
      f32x4 z = zero4();
      const float bb = sBeta[16 * b + lo];
#pragma unroll
      for (int c = a; c < b; ++c) {
        const float4 e4 = *reinterpret_cast<const float4*>(sEkk + (16 * b + lo) * SM + 16 * c + 4 * grp);
        const float av[4] = {bb * e4.x, bb * e4.y, bb * e4.z, bb * e4.w};
        z = mma16<true>(av, Xb[c], z);
      }
      float lv[4], zb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lv[r] = -sL[(16 * b + lo) * SM + 16 * b + 4 * grp + r];
        zb[r] = z[r];
      }
      const f32x4 xv = mma16<true>(lv, zb, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Xb[b][r] = xv[r];
        sL[(16 * b + 4 * grp + r) * SM + 16 * a + lo] = xv[r];
      }
    }
  }
  __syncthreads();

  // ---- dT = lowerIncl(dW (K Gamma)^T + dU V^T) into M3
  for (int t = wave; t < Cf::NPAIR; t += 8) {
    int tb, ta;
    tri_pair(t, tb, ta);
    const int r0 = 16 * tb, i0 = 16 * ta;
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    f32x4 acc = tile_mm4<F32, DK, true>(
        [&](int m, int k) { return ld4f(reinterpret_cast<const float4*>(&at(gr, GL::DW + (r0 + m) * DK + k))); },
        [&](int k, int n) {
          return mul4(ld4f(sK + (i0 + n) * SK + k), exp4(*reinterpret_cast<const float4*>(sG + (i0 + n) * SG + k), z4));
        },
        zero4());
    acc = tile_mm4<F32, DV, true, false>(  // v is exact in the operand type: only dU is split
        [&](int m, int k) { return ld4f(reinterpret_cast<const float4*>(&at(gr, GL::DU + (r0 + m) * DV + k))); },
        [&](int k, int n) { return v4_at(i0 + n, k); }, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * grp + r, col = i0 + lo;
      sM3[row * SM + col] = col <= row ? acc[r] : 0.f;
    }
  }
  for (int e = tid; e < C * C; e += NTH) {
    const int r = e / C, i = e - r * C;
    if ((i >> 4) > (r >> 4)) sM3[r * SM + i] = 0.f;
  }

  // ---- owned tiles: dKG = T^T dW (T = L diag(beta)); dK += dKG Gamma, dG += dKG K Gamma; and
  // dV = T^T dU, straight to the output.  With d_k = d_v the dV tile of the same row tile and column
  // tile index is formed beside each owned tile, the T^T fragments shared by the two products.
  constexpr bool DKV = NTK == NTV;
  f32x4 aq[MAXT], ak[MAXT], ag[MAXT];
#pragma unroll
  for (int q = 0; q < MAXT; ++q) {
    aq[q] = zero4();
    ak[q] = zero4();
    ag[q] = zero4();
    const int t = wave + 8 * q;
    if (t < NTILE) {
      const int i0 = 16 * tile_row(q, t), c0 = 16 * tile_col(t);
      auto ta = [&](int m, int k) { return sL[k * SM + i0 + m] * sBeta[i0 + m]; };
      auto bw = [&](int k, int n) { return at(gr, GL::DW + k * DK + c0 + n); };
      f32x4 d = zero4();
      if constexpr (DKV) {
        f32x4 v = zero4();
        tile_mm2<F32, C, true>(ta, bw, [&](int k, int n) { return at(gr, GL::DU + k * DV + c0 + n); }, d, v);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + 4 * grp + r;
          if constexpr (STG_V)
            reinterpret_cast<__bf16*>(sM4)[i * (DV + 8) + c0 + lo] = (__bf16)v[r];
          else if (i < nr)
            stg_at<F32>(dvb, (uint32_t)(i * H * DV + c0 + lo), v[r]);
        }
      } else {
        d = tile_mm<F32, C, true>(ta, bw, zero4());
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * grp + r, c = c0 + lo;
        const float gam = __expf(sG[i * SG + c]);
        ak[q][r] = d[r] * gam;
        ag[q][r] = d[r] * tf(sK[i * SK + c]) * gam;
      }
    }
  }
  if constexpr (!DKV) {
    for (int t = wave; t < Cf::NTC * NTV; t += 8) {
      const int i0 = 16 * (t / NTV), j0 = 16 * (t % NTV);
      const f32x4 d = tile_mm<F32, C, true>([&](int m, int k) { return sL[k * SM + i0 + m] * sBeta[i0 + m]; },
                                            [&](int k, int n) { return at(gr, GL::DU + k * DV + j0 + n); }, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * grp + r;
        if constexpr (STG_V)
          reinterpret_cast<__bf16*>(sM4)[i * (DV + 8) + j0 + lo] = (__bf16)d[r];
        else if (i < nr)
          stg_at<F32>(dvb, (uint32_t)(i * H * DV + j0 + lo), d[r]);
      }
    }
  }
  __syncthreads();
  if constexpr (STG_V) rows_out_bf16<C, DV, NTH>(reinterpret_cast<const __bf16*>(sM4), dvb, H, nr, tid);

  // ---- column part of dbeta (T = L diag(beta)) and dL = dT diag(beta): NPC lanes per column
  constexpr int NPC = NTH / C;
  {
    const int i = tid / NPC, u = tid - i * NPC;
    float s = 0.f;
    for (int r = u; r < C; r += NPC) {
      const float t = sM3[r * SM + i];
      s = fmaf(t, sL[r * SM + i], s);
      sM3[r * SM + i] = t * sBeta[i];
    }
    s = group_sum<NPC>(s);
    if (u == 0) sDb[i] = s;
  }
  __syncthreads();
  // ---- Y = L^T dL (into M4), MFMA tiles: Y[a][bb] = sum_r L[r][a] dL[r][bb]
  for (int t = wave; t < Cf::NTC * Cf::NTC; t += 8) {
    const int a0 = 16 * (t / Cf::NTC), b0 = 16 * (t % Cf::NTC);
    const f32x4 y = tile_mm<F32, C, true>([&](int m, int k) { return sL[k * SM + a0 + m]; },
                                          [&](int k, int n) { return sM3[k * SM + b0 + n]; }, zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) sM4[(a0 + 4 * grp + r) * SM + b0 + lo] = y[r];
  }
  __syncthreads();
  // ---- dA = strictLower(-Y L^T) (into M3): dA[a][bb] = -sum_s Y[a][s] L[bb][s], a > bb
  for (int t = wave; t < Cf::NTC * Cf::NTC; t += 8) {
    const int a0 = 16 * (t / Cf::NTC), b0 = 16 * (t % Cf::NTC);
    f32x4 d = zero4();
    if (b0 <= a0) {
      if constexpr (F32 || C % 32 == 0)
        d = tile_mm4<F32, C, true>([&](int m, int k) { return *reinterpret_cast<const float4*>(sM4 + (a0 + m) * SM + k); },
                                   [&](int k, int n) { return *reinterpret_cast<const float4*>(sL + (b0 + n) * SM + k); }, d);
      else
        d = tile_mm<F32, C, true>([&](int m, int k) { return sM4[(a0 + m) * SM + k]; },
                                  [&](int k, int n) { return sL[(b0 + n) * SM + k]; }, d);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = a0 + 4 * grp + r, bb = b0 + lo;
      sM3[a * SM + bb] = a > bb ? -d[r] : 0.f;
    }
  }
  __syncthreads();
  // ---- row part of dbeta (A = diag(beta) Ekk), dEkk = diag(beta) dA in place: NPC lanes per row;
  // dEqk = dP into M4
  {
    const int r = tid / NPC, u = tid - r * NPC;
    float s = 0.f;
    for (int i = u; i < r; i += NPC) {
      const float da = sM3[r * SM + i];
      s = fmaf(da, sEkk[r * SM + i], s);
      sM3[r * SM + i] = sBeta[r] * da;
    }
    s = group_sum<NPC>(s);
    if (u == 0 && r < nr) stg_at<F32>(dbb, (uint32_t)(r * H), sDb[r] + s);
  }
  for_units<C * C / 4, NTH>(tid, [&](int e) {  // 4 floats per access (records of grads are 256-byte aligned)
    const int r = (4 * e) / C, i = 4 * e - r * C;
    *reinterpret_cast<float4*>(sM4 + r * SM + i) = reinterpret_cast<const float4*>(gr + GL::DP)[e];
  });
  __syncthreads();

  // d(Q Gamma) and dKd of the owned elements, loaded here so that their latency passes behind the
  // Ekk/Eqk backward (they are used in the elementwise phase after it)
  float pfq[MAXT][4], pfk[MAXT][4];
#pragma unroll
  for (int q = 0; q < MAXT; ++q) {
    const int t = wave + 8 * q;
    if (t >= NTILE) continue;
    const int r0 = 16 * tile_row(q, t), c = 16 * tile_col(t) + lo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r0 + 4 * grp + r;
      pfq[q][r] = at(gr, GL::DQG + i * DK + c);
      pfk[q][r] = at(gr, GL::DKD + i * DK + c);
    }
  }
  // ---- through Ekk and Eqk, on the owned tiles (rows r0.., channels c0..):
  //   row side (reference R = G before the row tile):
  //     dQe = e^{G_r - R} sum_{i <= r} dEqk[r][i] (K e^{R - G})[i],   dKr = the same with dEkk
  //     dQ += dQe, dK += dKr, dG += q dQe + k dKr
  //   column side (reference R' = G at the tile's last row):
  //     dKc = e^{R' - G_i} sum_{r >= i} (dEqk[r][i] q_r + dEkk[r][i] k_r) e^{G_r - R'}
  //     dK += dKc, dG -= k dKc
  // (dEqk is lower-inclusive, dEkk strictly lower: both zero elsewhere)
#pragma unroll
  for (int q = 0; q < MAXT; ++q) {
    const int t = wave + 8 * q;
    if (t >= NTILE) continue;
    const int r0 = 16 * tile_row(q, t), c = 16 * tile_col(t) + lo;
    const float R = r0 > 0 ? sG[(r0 - 1) * SG + c] : 0.f, R2 = sG[(r0 + 15) * SG + c];
    // fp32 MFMA (16x16x4) for both input types: with bf16 inputs the operands built here (an exponent
    // factor per element) would otherwise be split into bf16 hi + lo parts element by element for
    // three bf16 products; the fp32 products are exact in the operands and took this phase from
    // 0.20 to 0.16 ms per 4 x 16 x 4096 backward call
    using OF = Op<true>;
    f32x4 d1 = zero4(), d2 = zero4(), d3 = zero4();
#pragma unroll EEU
    for (int s = 0; s < OF::nks(r0 + 16); ++s) {
      const int k = OF::kidx(s, grp, 0);
      const float fb = tf(sK[k * SK + c]) * __expf(R - sG[k * SG + c]);
      d1 = OF::mma(sM4[(r0 + lo) * SM + k], fb, d1);
      d2 = OF::mma(sM3[(r0 + lo) * SM + k], fb, d2);
    }
#pragma unroll EEU
    for (int s = 0; s < OF::nks(C - r0); ++s) {
      const int r = r0 + OF::kidx(s, grp, 0);
      const float e = __expf(sG[r * SG + c] - R2);
      d3 = OF::mma(sM4[r * SM + r0 + lo], q_at(r, c) * e, d3);
      d3 = OF::mma(sM3[r * SM + r0 + lo], tf(sK[r * SK + c]) * e, d3);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r0 + 4 * grp + r;
      const float G = sG[i * SG + c], qv = q_at(i, c), kv = tf(sK[i * SK + c]);
      const float f = __expf(G - R), f2 = __expf(R2 - G);
      const float dqe = d1[r] * f, dkr = d2[r] * f, dkc = d3[r] * f2;
      aq[q][r] += dqe;
      ak[q][r] += dkr + dkc;
      ag[q][r] += qv * dqe + kv * (dkr - dkc);
    }
  }

  // ---- elementwise: Q Gamma, Kd = K e^{gl - G}, and the chunk's total decay gl
#pragma unroll
  for (int q = 0; q < MAXT; ++q) {
    const int t = wave + 8 * q;
    if (t >= NTILE) continue;
    const int tm = tile_row(q, t), r0 = 16 * tm, c = 16 * tile_col(t) + lo;
    const float gl = sG[(C - 1) * SG + c];
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r0 + 4 * grp + r;
      const float G = sG[i * SG + c], gam = __expf(G), dec = __expf(gl - G);
      const float qv = q_at(i, c), kv = tf(sK[i * SK + c]);
      const float dqg = pfq[q][r], dkd = pfk[q][r];
      aq[q][r] = fmaf(dqg, gam, aq[q][r]);
      ag[q][r] = fmaf(dqg * qv, gam, ag[q][r]);
      ak[q][r] = fmaf(dkd, dec, ak[q][r]);
      const float tt = dkd * kv * dec;
      ag[q][r] -= tt;
      part += tt;
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (grp == 0) sRed[tm * DK + c] = part;
  }
  __syncthreads();
  if (tid < DK) {
    float s = at(gr, GL::DGL + tid);
    for (int o = 0; o < Cf::NTC; ++o) s += sRed[o * DK + tid];
    sDgl[tid] = s;
  }
  __syncthreads();  // sG (G) is read for the last time above
#pragma unroll
  for (int q = 0; q < MAXT; ++q) {
    const int t = wave + 8 * q;
    if (t >= NTILE) continue;
    const int r0 = 16 * tile_row(q, t), c = 16 * tile_col(t) + lo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r0 + 4 * grp + r;
      float dg = ag[q][r];
      if (i == C - 1) dg += sDgl[c];
      sG[i * SG + c] = dg;
      if constexpr (STG_QK) {
        reinterpret_cast<__bf16*>(sEkk)[i * (DK + 8) + c] = (__bf16)aq[q][r];
        reinterpret_cast<__bf16*>(sL)[i * (DK + 8) + c] = (__bf16)ak[q][r];
      } else if (i < nr) {
        stg_at<F32>(dqb, (uint32_t)(i * H * DK + c), aq[q][r]);
        stg_at<F32>(dkb, (uint32_t)(i * H * DK + c), ak[q][r]);
      }
    }
  }
  __syncthreads();
  if constexpr (STG_QK) {
    rows_out_bf16<C, DK, NTH>(reinterpret_cast<const __bf16*>(sEkk), dqb, H, nr, tid);
    rows_out_bf16<C, DK, NTH>(reinterpret_cast<const __bf16*>(sL), dkb, H, nr, tid);
  }
  // ---- dg = reverse cumulative sum of dG over the chunk's rows, written 8 channels per access
  scan_rows<DK, C, Cf::NPART, Cf::RPP, true>(sG, SG, sScan, tid);
  if constexpr (F32) {
    for (int e = tid; e < C * DK; e += NTH) {
      const int r = e / DK, c = e - r * DK;
      if (r < nr) stg_at<F32>(dgb, (uint32_t)(r * H * DK + c), sG[r * SG + c]);
    }
  } else {
    for_units<C * DK / 8, NTH>(tid, [&](int e) {
      const int r = (8 * e) / DK, c = 8 * e - r * DK;
      if (r < nr) {
        const float4 a = *reinterpret_cast<const float4*>(sG + r * SG + c), b = *reinterpret_cast<const float4*>(sG + r * SG + c + 4);
        at(static_cast<uint4*>(dgb), (uint32_t)((r * H * DK + c) / 8)) =
            make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
      }
    });
  }
}

// ------------------------------------------------------------------------------------------------
#define KDA_BWD_INSTANCES(X)                                                                    \
  X(false, 64, 64, 16) X(false, 64, 64, 32) X(false, 64, 64, 64)                                \
  X(false, 64, 128, 16) X(false, 64, 128, 32) X(false, 64, 128, 64)                             \
  X(false, 128, 64, 16) X(false, 128, 64, 32) X(false, 128, 64, 64)                             \
  X(false, 128, 128, 16) X(false, 128, 128, 32) X(false, 128, 128, 64)                          \
  X(true, 64, 64, 16) X(true, 64, 64, 32) X(true, 64, 64, 64)                                   \
  X(true, 64, 128, 16) X(true, 64, 128, 32) X(true, 64, 128, 64)                                \
  X(true, 128, 64, 16) X(true, 128, 64, 32) X(true, 128, 64, 64)                                \
  X(true, 128, 128, 16) X(true, 128, 128, 32) X(true, 128, 128, 64)

bool chunked_backward_supported(bool f32, int dk, int dv, int chunk) {
#define KDA_SUP(F, D, V, CC) \
  if (f32 == F && dk == D && dv == V && chunk == CC) return record_bytes(f32, dk, dv, chunk) > 0;
  KDA_BWD_INSTANCES(KDA_SUP)
#undef KDA_SUP
  return false;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t grad_floats(int dk, int dv, int chunk) {
  const int64_t f = (int64_t)chunk * dv + (int64_t)chunk * chunk + 3 * (int64_t)chunk * dk + dk;
  return (size_t)((f + 63) & ~(int64_t)63);
}

// Segments of the adjoint chain, as the forward chain's: when (sequence, head, 32-column slice)
// alone would leave compute units idle, every sequence is split into nseg segments of at least 32
// chunks (at most 64 segments); one workgroup per (sequence, head, segment, slice).
struct BwdPlan {
  int nseg, seg_len;
};
static BwdPlan bwd_plan(int64_t units, int nch, int dv) {
  BwdPlan pl{1, 0};
  const int64_t per = units * (dv / 32);
  const int cus = compute_units();
  if (per < cus && nch >= 64) {
    int64_t nseg = (cus + per - 1) / per;
    if (nseg > nch / 32) nseg = nch / 32;
    if (nseg > 64) nseg = 64;
    if (nseg >= 2) {
      pl.seg_len = (int)((nch + nseg - 1) / nseg);
      pl.nseg = (nch + pl.seg_len - 1) / pl.seg_len;
    }
  }
  return pl;
}

// The chunks of B equal-length sequences, or a bound on those of num_seqs packed ones (each sequence
// adds at most one partial chunk), as the forward counts them.
static int64_t bwd_max_chunks(int C, int num_seqs, int T, bool varlen) {
  return varlen ? (int64_t)T / C + num_seqs : (int64_t)num_seqs * ((T + C - 1) / C);
}

// The backward's buffers, each 256-byte aligned.  The part a forward leaves for it: [forward
// workspace: records (and, packed, the chunk map)][states: chunks H dk dv].  The backward's own:
// [dstates: chunks H dk dv][grads: chunks H GradLayout floats][o scratch: tokens H dv elements,
// only where the forward is recomputed], and for a segmented adjoint chain [segment end adjoints:
// units nseg dk dv fp32][summaries: units (nseg - 1) dk (dv + dk) fp32].  States and adjoints are
// in the operand type (fp32 or bf16).  tokens: B T, or T_total for packed sequences.
struct BwdSizes {
  size_t fwd = 0, st = 0, gr = 0, os = 0, seg_end = 0, seg_sum = 0;
};
static BwdSizes bwd_sizes(bool f32, int dk, int dv, int chunk, int num_seqs, int T, int H, bool varlen) {
  BwdSizes z;
  const int64_t mc = bwd_max_chunks(chunk, num_seqs, T, varlen), units = (int64_t)num_seqs * H, items = mc * H;
  const int64_t tokens = varlen ? (int64_t)T : (int64_t)num_seqs * T;
  z.fwd = al256(chunked_forward_workspace(f32, dk, dv, chunk, mc, H, num_seqs, varlen));
  z.st = al256((size_t)items * dk * dv * (f32 ? 4 : 2));
  z.gr = al256((size_t)items * grad_floats(dk, dv, chunk) * 4);
  z.os = al256((size_t)tokens * H * dv * (f32 ? 4 : 2));
  if (!varlen) {
    const BwdPlan pl = bwd_plan(units, (T + chunk - 1) / chunk, dv);
    if (pl.nseg > 1) {
      z.seg_end = al256((size_t)(units * pl.nseg) * dk * dv * 4);
      z.seg_sum = al256((size_t)(units * (pl.nseg - 1)) * dk * (dv + dk) * 4);
    }
  }
  return z;
}

size_t chunked_backward_workspace(bool f32, int dk, int dv, int chunk, int num_seqs, int T, int H, bool varlen) {
  if (!chunked_backward_supported(f32, dk, dv, chunk)) return 0;
  const BwdSizes z = bwd_sizes(f32, dk, dv, chunk, num_seqs, T, H, varlen);
  return z.fwd + 2 * z.st + z.gr + z.os + z.seg_end + z.seg_sum;
}

size_t chunked_backward_saved_bytes(bool f32, int dk, int dv, int chunk, int num_seqs, int T, int H, bool varlen) {
  if (!chunked_backward_supported(f32, dk, dv, chunk)) return 0;
  const BwdSizes z = bwd_sizes(f32, dk, dv, chunk, num_seqs, T, H, varlen);
  return z.fwd + z.st;
}

size_t chunked_backward_own_bytes(bool f32, int dk, int dv, int chunk, int num_seqs, int T, int H, bool varlen) {
  if (!chunked_backward_supported(f32, dk, dv, chunk)) return 0;
  const BwdSizes z = bwd_sizes(f32, dk, dv, chunk, num_seqs, T, H, varlen);
  return z.st + z.gr + z.seg_end + z.seg_sum;
}

template <bool F32, int DK, int DV, int C>
static hipError_t launch_backward_kernels(const BwdParams& p, int64_t units, void* stream) {
  static_assert(GradLayout<DK, DV, C>::FLOATS == (((int64_t)C * DV + C * C + 3 * C * DK + DK + 63) & ~(int64_t)63),
                "grad layout");
  hipError_t e = hipSuccess;
  // bf16 records of 32- or 64-token chunks: the accumulator-resident adjoint chain
  constexpr bool TR = !F32 && C >= 32;
  if (p.nseg > 1) {  // segment summaries, then every segment's end adjoint from dhT
    const int64_t su = units * (p.nseg - 1);
    const dim3 grid((unsigned)(((su + 7) / 8) * 8 * ((DV + DK) / 32)));
    if constexpr (TR) hipLaunchKernelGGL((bwd_chain_t_kernel<DK, DV, C, true>), grid, dim3(384), 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL((bwd_chain_kernel<F32, DK, DV, C, true>), grid, dim3(512), 0, (hipStream_t)stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_segment_combine(p.dhT, p.bsend, const_cast<float*>(p.bstart), (int)units, p.nseg, DK, DV, stream)) !=
        hipSuccess)
      return e;
  }
  const int64_t su = units * p.nseg;
  const dim3 grid((unsigned)(((su + 7) / 8) * 8 * (DV / 32)));
  if constexpr (TR) hipLaunchKernelGGL((bwd_chain_t_kernel<DK, DV, C, false>), grid, dim3(384), 0, (hipStream_t)stream, p);
  else hipLaunchKernelGGL((bwd_chain_kernel<F32, DK, DV, C, false>), grid, dim3(512), 0, (hipStream_t)stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.items == 0) return e;
  hipLaunchKernelGGL((bwd_state_kernel<F32, DK, DV, C>), dim3((unsigned)p.items), dim3(512), 0, (hipStream_t)stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_intra_kernel<F32, DK, DV, C>), dim3((unsigned)p.items), dim3(512), 0, (hipStream_t)stream, p);
  return hipGetLastError();
}

// The forward as the backward needs it: the state after every full chunk kept at that chunk's
// record slot (the start state of the sequence's next chunk), in the operand type.
static hipError_t forward_for_backward(const BackwardArgs& a, unsigned char* ws, size_t fwd_bytes, void* states,
                                       void* o, float* hT) {
  PrefillArgs f;
  f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.beta = a.beta;
  f.h0 = a.h0; f.o = o; f.hT = hT;
  f.cu_seqlens = a.cu_seqlens; f.num_seqs = a.B; f.T = a.T;
  f.H = a.H; f.dk = a.dk; f.dv = a.dv; f.chunk = a.chunk; f.f32 = a.f32;
  f.workspace = ws; f.workspace_bytes = fwd_bytes; f.stream = a.stream;
  f.states = static_cast<float*>(states);  // fp32 or bf16 elements (f.states_bf16)
  f.state_every = a.chunk;
  f.states_by_chunk = true;
  f.states_bf16 = !a.f32;
  return launch_chunked_forward(f);
}

hipError_t launch_forward_train(const BackwardArgs& a, void* saved, void* o, float* hT) {
  if (!chunked_backward_supported(a.f32, a.dk, a.dv, a.chunk)) return hipErrorInvalidValue;
  const BwdSizes z = bwd_sizes(a.f32, a.dk, a.dv, a.chunk, a.B, a.T, a.H, a.cu_seqlens != nullptr);
  unsigned char* sv = static_cast<unsigned char*>(saved);
  return forward_for_backward(a, sv, z.fwd, sv + z.fwd, o, hT);
}

hipError_t launch_chunked_backward(const BackwardArgs& a) {
  if (!chunked_backward_supported(a.f32, a.dk, a.dv, a.chunk)) return hipErrorInvalidValue;
  const bool varlen = a.cu_seqlens != nullptr;
  const int C = a.chunk, nch = varlen ? 0 : (a.T + C - 1) / C;
  const int64_t mc = bwd_max_chunks(C, a.B, a.T, varlen), units = (int64_t)a.B * a.H, items = mc * a.H;
  const int64_t tokens = varlen ? (int64_t)a.T : (int64_t)a.B * a.T;
  const BwdPlan pl = varlen ? BwdPlan{1, 0} : bwd_plan(units, nch, a.dv);
  if (units <= 0 || (units * pl.nseg + 7) * ((a.dv + a.dk) / 32) > INT32_MAX || items > INT32_MAX)
    return hipErrorInvalidValue;
  const BwdSizes z = bwd_sizes(a.f32, a.dk, a.dv, C, a.B, a.T, a.H, varlen);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  // the forward's part: from a forward-train call, or recomputed at the start of the workspace
  unsigned char* saved = a.saved ? static_cast<unsigned char*>(const_cast<void*>(a.saved)) : ws;
  unsigned char* own = a.saved ? ws : ws + z.fwd + z.st;
  void* states = saved + z.fwd;
  void* dstates = own;
  float* grads = reinterpret_cast<float*>(own + z.st);
  unsigned char* seg = own + z.st + z.gr + (a.saved ? 0 : z.os);
  hipError_t e = hipSuccess;
  if (!a.saved && tokens > 0) {
    if ((e = forward_for_backward(a, ws, z.fwd, states, own + z.st + z.gr, nullptr)) != hipSuccess) return e;
  }
  BwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta; p.dO = a.dO;
  p.h0 = a.h0; p.dhT = a.dhT;
  p.records = saved; p.states = states; p.dstates = dstates; p.grads = grads;
  p.dq = a.dq; p.dk = a.dk_out; p.dv = a.dv_out; p.dg = a.dg; p.dbeta = a.dbeta; p.dh0 = a.dh0;
  p.T = a.T; p.H = a.H; p.nch = nch; p.units = (int)units; p.items = items;
  p.cu = a.cu_seqlens; p.num_seqs = a.B;
  p.chunk0 = p.order = nullptr;
  if (varlen) {
    int32_t *c0, *ord;
    chunk_map_of(saved, a.f32, a.dk, a.dv, C, mc, a.H, a.B, &c0, &ord);
    // built by the forward recompute; with no tokens every sequence is empty and only the map is needed
    if (tokens == 0 && (e = launch_chunk_map(a.cu_seqlens, a.B, a.T, C, c0, ord, a.stream)) != hipSuccess) return e;
    p.chunk0 = c0;
    p.order = ord;
  }
  p.nseg = pl.nseg; p.seg_len = pl.seg_len;
  p.bstart = reinterpret_cast<const float*>(seg);
  p.bsend = reinterpret_cast<float*>(seg + al256((size_t)(units * pl.nseg) * a.dk * a.dv * 4));
#define KDA_BWD_LAUNCH(F, D, V, CC) \
  if (a.f32 == F && a.dk == D && a.dv == V && C == CC) return launch_backward_kernels<F, D, V, CC>(p, units, a.stream);
  KDA_BWD_INSTANCES(KDA_BWD_LAUNCH)
#undef KDA_BWD_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace kda
